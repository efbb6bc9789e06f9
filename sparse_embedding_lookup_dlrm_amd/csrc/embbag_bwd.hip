// Sparse backward of the embedding-bag + interaction forward, then SGD on the
// touched rows, for gfx950. All kernels are enqueued on one stream with no host
// synchronisation; the number of distinct rows stays on the device.
//
// 1. interaction backward: the gradient of Z[i].Z[j] with respect to Z[i] is
//    Z[j], so dZ[b] = S[b] Z[b] with S[b] the symmetric F x F matrix holding the
//    upstream gradient of pair (i, j) at (i, j) and (j, i), zero diagonal;
//    dL/dpooled[b][t] = dZ[b][1 + t], dL/de0[b] = d_out[b][:D] + dZ[b][0].
//    One workgroup per sample; in the sparse backward these workgroups ride as
//    extras on the sort's scatter launches and the segment build (or on the
//    per-table sort's first launch), since nothing before the reduce reads dZ.
// 2. keys: occurrence p of bag (t, b) gets key base_t + index (its global row)
//    and value p; an out-of-range index, or a position no bag covers (invalid
//    offsets), gets the sentinel key sum(rows).
// 3. stable LSD radix sort of (key, p), 8 or 9 bits per pass (9 only where
//    that saves a pass): per-tile digit counts, each tile's digit offsets (from
//    the digit-major count table, summed inside the scatter for up to 128
//    tiles, else scanned per digit by one kernel), a stable scatter that ranks
//    equal digits inside a wave with ballots. The last pass also writes each
//    sorted position's bag.
//    Small batches (at most one tile of occurrences per table on average) sort
//    per table instead: a table's occurrences form one range of positions and
//    one range of keys, so one workgroup per table sorts its range by row
//    index and a second launch places the ranges (table_sort, table_place):
//    two launches in place of the key build and two or three per radix pass.
// 4. segments (API outputs only): head flags (key differs from its
//    predecessor), scanned into the position of each distinct key. With few
//    reduce chunks the reduce counts each chunk's heads and the combine step
//    writes the outputs (no launches of their own).
// 5. segmented sums of the rows dL/dpooled over the sorted occurrences, in
//    fixed chunks of positions whatever the segment lengths (a fixed order, so
//    the result is deterministic), then W <- W - lr * G in fp32, rounded once
//    to the table's storage type (or the row-wise AdaGrad step).
#include <algorithm>

#include "scan_impl.h"

namespace dlrm {

constexpr int kBwdThreads = 256;
// Digits of 8 bits, or 9 where that takes one pass fewer (keys of 9, 17-18 or
// 25-27 bits): a 9-bit digit has 512 bins, two per thread.
constexpr int kMaxRadixBits = 9;
constexpr int kMaxRadixBins = 1 << kMaxRadixBits;
constexpr int kRadixPerThread = 8;
constexpr int kRadixTile = kBwdThreads * kRadixPerThread;  // 2048 keys per tile
constexpr int kRadixWaves = kBwdThreads / kWave;
constexpr int kRadixRounds = kRadixTile / kRadixWaves / kWave;  // rounds of 64 keys per wave

// ---------------------------------------------------------------------------
// 1. interaction backward
// ---------------------------------------------------------------------------
// With self-pairs the pair (i, i) sits at i(i+1)/2 + i and its gradient counts
// twice on the diagonal of S (d(Z_i . Z_i)/dZ_i = 2 Z_i).
//
// Sample b's interaction backward by one workgroup, with smem holding
// F*(D+4) + Fp*F floats. The standalone kernel runs one sample per workgroup;
// inside the sparse backward the samples are shared out as extra workgroups
// of the key build and sort launches (IbwdShare), whose own few workgroups
// leave most of the chip idle, so this work overlaps the sort's chain of
// launches instead of running before it.
struct IbwdShare {
  int T, D;
  bool self_pairs;  // pairs i >= j (else i > j)
  bool with_emb;    // d_out holds the gradient of every Z row ahead of the pair gradients
  const float* e0;
  const float* pooled;
  const float* d_out;
  float* d_pooled;
  float* d_e0;
  int first;  // the sample of the first extra workgroup
  int count;  // extra workgroups (samples) of this launch
};

__device__ __forceinline__ void interact_bwd_sample(const IbwdShare& ia, int b, float* smem) {
  const int T = ia.T, D = ia.D;
  const bool self_pairs = ia.self_pairs;
  const bool with_emb = ia.with_emb;
  const float* __restrict__ e0 = ia.e0;
  const float* __restrict__ pooled = ia.pooled;
  const float* __restrict__ d_out = ia.d_out;
  float* __restrict__ d_pooled = ia.d_pooled;
  float* __restrict__ d_e0 = ia.d_e0;
  const int F = T + 1;
  const int LD = D + 4;
  const int dot0 = with_emb ? F * D : D;  // first pair gradient of a sample's row of d_out
  const int W = dot0 + (self_pairs ? F * (F + 1) / 2 : F * (F - 1) / 2);
  const int Fp = (F + 3) & ~3;    // S rows, padded with zeros to whole blocks of 4
  float* Z = smem;                // [F][LD]
  float* S = smem + F * LD;       // [Fp][F]
  const int D4 = D / 4;
  // Z and S are filled in batches whose loads are all issued before the first
  // LDS store, so a batch costs one memory round trip, not one per element; the
  // first batch of S and the e0 gradient are loaded before Z's batches
  constexpr int kBatch = 4;
  const float* g = d_out + static_cast<size_t>(b) * W + dot0;
  auto s_value = [&](int i) -> float {  // S[r][c] from the upstream pair gradients (i = r * F + c)
    const int r = i / F, c = i - r * F;
    const int hi = r > c ? r : c, lo = r > c ? c : r;
    const bool use = i < F * F && (self_pairs || hi != lo);
    const int k = self_pairs ? hi * (hi + 1) / 2 + lo : hi * (hi - 1) / 2 + lo;
    float v = g[use ? k : 0];
    if (!use) v = 0.f;
    else if (self_pairs && hi == lo) v *= 2.f;
    return v;
  };
  float s_first[kBatch];
#pragma unroll
  for (int u = 0; u < kBatch; ++u) s_first[u] = s_value(threadIdx.x + u * kBwdThreads);
  // the upstream gradient of e0 (row 0 is item threadIdx.x < D/4 of the dZ loop)
  float4 go = make_float4(0.f, 0.f, 0.f, 0.f);
  if (d_e0 && static_cast<int>(threadIdx.x) < D4) {
    const float* p = d_out + static_cast<size_t>(b) * W + 4 * threadIdx.x;
    go = make_float4(p[0], p[1], p[2], p[3]);
  }
  for (int i0 = threadIdx.x; i0 < F * D4; i0 += kBatch * kBwdThreads) {
    float4 v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = i0 + u * kBwdThreads;
      const int ic = i < F * D4 ? i : i0;  // past the end: reload the first element (in bounds)
      const int f = ic / D4, d = (ic - f * D4) * 4;
      v[u] = f == 0 ? *reinterpret_cast<const float4*>(e0 + static_cast<size_t>(b) * D + d)
                    : *reinterpret_cast<const float4*>(pooled + (static_cast<size_t>(b) * T + f - 1) * D + d);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = i0 + u * kBwdThreads;
      if (i < F * D4) {
        const int f = i / D4, d = (i - f * D4) * 4;
        *reinterpret_cast<float4*>(Z + f * LD + d) = v[u];
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kBatch; ++u) {
    const int i = threadIdx.x + u * kBwdThreads;
    if (i < Fp * F) S[i] = s_first[u];
  }
  for (int i0 = threadIdx.x + kBatch * kBwdThreads; i0 < Fp * F; i0 += kBatch * kBwdThreads) {
    float v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) v[u] = s_value(i0 + u * kBwdThreads);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = i0 + u * kBwdThreads;
      if (i < Fp * F) S[i] = v[u];
    }
  }
  __syncthreads();
  // dZ = S Z: a thread computes 4 rows (f0..f0+3) of one float4 column, so each
  // Z read serves 4 rows; the lanes of a wave share f0 (the column varies
  // fastest), so their S reads are broadcasts
  for (int i = threadIdx.x; i < (Fp / 4) * D4; i += kBwdThreads) {
    const int fb = i / D4, d = (i - fb * D4) * 4;
    const int f0 = 4 * fb;
    float4 acc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = make_float4(0.f, 0.f, 0.f, 0.f);
    const float* srow = S + f0 * F;
    for (int j = 0; j < F; ++j) {
      const float4 z = *reinterpret_cast<const float4*>(Z + j * LD + d);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float s = srow[r * F + j];
        acc[r].x = fmaf(s, z.x, acc[r].x);
        acc[r].y = fmaf(s, z.y, acc[r].y);
        acc[r].z = fmaf(s, z.z, acc[r].z);
        acc[r].w = fmaf(s, z.w, acc[r].w);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int f = f0 + r;
      if (f == 0) {
        if (d_e0) {
          *reinterpret_cast<float4*>(d_e0 + static_cast<size_t>(b) * D + d) =
              make_float4(go.x + acc[r].x, go.y + acc[r].y, go.z + acc[r].z, go.w + acc[r].w);
        }
      } else if (f < F) {
        float4 v = acc[r];
        if (with_emb) {  // the direct gradient of the pooled row, which is in the output too
          const float4 dir = *reinterpret_cast<const float4*>(d_out + static_cast<size_t>(b) * W + f * D + d);
          v = make_float4(v.x + dir.x, v.y + dir.y, v.z + dir.z, v.w + dir.w);
        }
        *reinterpret_cast<float4*>(d_pooled + (static_cast<size_t>(b) * T + f - 1) * D + d) = v;
      }
    }
  }
}

__global__ __launch_bounds__(kBwdThreads) void interact_bwd_kernel(IbwdShare ia) {
  extern __shared__ __align__(16) float smem[];
  interact_bwd_sample(ia, ia.first + xcd_block(blockIdx.x, gridDim.x), smem);
}

// In a launch with own_blocks workgroups of its own: the extra workgroups take
// samples ia.first + (blockIdx.x - own_blocks). Returns true for those.
__device__ __forceinline__ bool ibwd_extra(const IbwdShare& ia, int own_blocks) {
  if (static_cast<int>(blockIdx.x) < own_blocks) return false;
  extern __shared__ __align__(16) float smem[];
  interact_bwd_sample(ia, ia.first + static_cast<int>(blockIdx.x) - own_blocks, smem);
  return true;
}

// ---------------------------------------------------------------------------
// 2. keys (a group of lanes per bag, table-major bag order = CSR order)
// ---------------------------------------------------------------------------
// LG lanes per bag (a power of two, 1..64): lane k of a bag's group handles
// its occurrences k, k + LG, ... so loads and stores are contiguous across the
// group; LG follows the average bag length.
template <int LG>
__global__ __launch_bounds__(kBwdThreads) void build_keys(MutTableArgs tabs, int T, int B, const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ indices, long long nnz,
                                                          int32_t sentinel, int32_t* __restrict__ keys,
                                                          int32_t* __restrict__ vals, int32_t* __restrict__ bag_of,
                                                          int32_t* status, int own_blocks, IbwdShare ia) {
  if (ibwd_extra(ia, own_blocks)) return;
  const long long g = static_cast<long long>(blockIdx.x) * kBwdThreads + threadIdx.x;
  const long long j = g / LG;
  const int sub = static_cast<int>(g % LG);
  if (j >= static_cast<long long>(T) * B) return;
  const int t = static_cast<int>(j / B), b = static_cast<int>(j - static_cast<long long>(t) * B);
  long long s0 = offsets[j], s1 = offsets[j + 1];
  bool bad_off = false;
  if (j == 0 && s0 != 0) bad_off = true;
  if (j == static_cast<long long>(T) * B - 1 && s1 != nnz) bad_off = true;
  if (s0 < 0) { s0 = 0; bad_off = true; }
  if (s0 > nnz) { s0 = nnz; bad_off = true; }
  if (s1 < 0) { s1 = 0; bad_off = true; }
  if (s1 > nnz) { s1 = nnz; bad_off = true; }
  // Bag j writes its range [o_j, max(o_j, o_j+1)) once clamped into [0, nnz].
  // For a valid CSR the ranges tile [0, nnz). With invalid offsets (flagged)
  // two things can happen. The positions before the first offset or from the
  // last offset on belong to no bag: the first and the last bag give them the
  // sentinel key. And where offsets decrease, the ranges of non-adjacent bags
  // can overlap; a position covered twice then ends up with either bag's key
  // (unspecified, as the header states), but every key written is in range.
  auto fill_gap = [&](long long g0, long long g1) {
    for (long long p = g0 + sub; p < g1; p += LG) {
      keys[p] = sentinel;
      vals[p] = static_cast<int32_t>(p);
      bag_of[p] = 0;
    }
  };
  if (j == 0) fill_gap(0, s0);
  if (j == static_cast<long long>(T) * B - 1) fill_gap(s1, nnz);
  if (s1 < s0) { s1 = s0; bad_off = true; }
  if (bad_off && sub == 0) flag(status, DLRM_STATUS_BAD_OFFSETS);
  const int rows = tabs.rows[t], base = tabs.base[t];
  const int bag = b * T + t;
  bool bad_idx = false;
  // four index loads in flight per step (past the bag: re-read its first index)
  constexpr int U = 4;
  for (long long p0 = s0 + sub; p0 < s1; p0 += U * LG) {
    int r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) r[u] = indices[p0 + u * LG < s1 ? p0 + u * LG : s0];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long long p = p0 + u * LG;
      if (p < s1) {
        int key = sentinel;
        if (r[u] >= 0 && r[u] < rows) key = base + r[u];
        else bad_idx = true;
        keys[p] = key;
        vals[p] = static_cast<int32_t>(p);
        bag_of[p] = bag;
      }
    }
  }
  if (bad_idx) flag(status, DLRM_STATUS_BAD_INDEX);
}

// ---------------------------------------------------------------------------
// 3. radix sort
// ---------------------------------------------------------------------------
template <int BITS>
__global__ __launch_bounds__(kBwdThreads) void radix_count(const int32_t* __restrict__ keys, long long n, int shift,
                                                           int ntiles, int32_t* __restrict__ counts, IbwdShare ia) {
  constexpr int kBins = 1 << BITS;
  if (ibwd_extra(ia, ntiles)) return;
  __shared__ int hist[kBins];
  for (int d = threadIdx.x; d < kBins; d += kBwdThreads) hist[d] = 0;
  __syncthreads();
  const long long base = static_cast<long long>(blockIdx.x) * kRadixTile;
#pragma unroll
  for (int k = 0; k < kRadixPerThread; ++k) {
    const long long i = base + k * kBwdThreads + threadIdx.x;
    if (i < n) atomicAdd(&hist[(static_cast<uint32_t>(keys[i]) >> shift) & (kBins - 1)], 1);
  }
  __syncthreads();
  for (int d = threadIdx.x; d < kBins; d += kBwdThreads) counts[static_cast<long long>(d) * ntiles + blockIdx.x] = hist[d];
}

// Up to this many tiles, each scatter workgroup works out its own digit
// offsets from the count table instead of a device-wide scan.
constexpr int kInlineScanTiles = 128;

// Where this tile's keys of each digit start in the output (gbase[d]): all
// keys of smaller digits, plus the keys of digit d in earlier tiles. Thread
// threadIdx.x handles digits threadIdx.x + j * 256. The count table is
// digit-major ([digit][tile]). With row_prefix null the digit's row is summed
// here; otherwise row_prefix holds each row's exclusive scan and row_total
// each row's sum (radix_row_scan). The digit totals are then scanned across
// the workgroup in digit order. lds holds kRadixWaves ints per digit per thread.
template <int BITS>
__device__ __forceinline__ void tile_digit_base(const int32_t* __restrict__ counts,
                                                const int32_t* __restrict__ row_prefix,
                                                const int32_t* __restrict__ row_total, int ntiles, int* lds,
                                                int* gbase) {
  constexpr int kDPT = (1 << BITS) / kBwdThreads;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  int tot[kDPT], pre[kDPT], x[kDPT];
#pragma unroll
  for (int j = 0; j < kDPT; ++j) {
    const int d = threadIdx.x + j * kBwdThreads;
    tot[j] = 0;
    pre[j] = 0;
    if (row_prefix) {
      pre[j] = row_prefix[static_cast<long long>(d) * ntiles + blockIdx.x];
      tot[j] = row_total[d];
    } else {
      const int32_t* row = counts + static_cast<long long>(d) * ntiles;
      for (int t0 = 0; t0 < ntiles; t0 += 8) {
        int c[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) c[u] = t0 + u < ntiles ? row[t0 + u] : 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          tot[j] += c[u];
          if (t0 + u < static_cast<int>(blockIdx.x)) pre[j] += c[u];
        }
      }
    }
    x[j] = tot[j];  // inclusive scan of the totals over the wave, then across the 4 waves
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(x[j], o, kWave);
      if (lane >= o) x[j] += y;
    }
    if (lane == kWave - 1) lds[j * kRadixWaves + wave] = x[j];
  }
  __syncthreads();
  int carry = 0;  // keys of all digits below threadIdx.x + j * 256's block of 256
#pragma unroll
  for (int j = 0; j < kDPT; ++j) {
    int before = carry;
    for (int w = 0; w < kRadixWaves; ++w) {
      const int v = lds[j * kRadixWaves + w];
      if (w < wave) before += v;
      carry += v;
    }
    gbase[threadIdx.x + j * kBwdThreads] = before + x[j] - tot[j] + pre[j];
  }
}

// Each digit's row of the count table (one workgroup per digit): exclusive
// scan across the tiles into row_prefix, and the row's sum into row_total.
__global__ __launch_bounds__(kScanThreads) void radix_row_scan(const int32_t* __restrict__ counts, int ntiles,
                                                               int32_t* __restrict__ row_prefix,
                                                               int32_t* __restrict__ row_total) {
  __shared__ long long lds[kScanThreads / kWave];
  const long long r0 = static_cast<long long>(blockIdx.x) * ntiles;
  long long carry = 0;
  for (int base = 0; base < ntiles; base += kScanChunk) {
    const int c0 = base + threadIdx.x * kScanPerThread;
    int v[kScanPerThread];
    long long sum = 0;
#pragma unroll
    for (int k = 0; k < kScanPerThread; ++k) {
      v[k] = c0 + k < ntiles ? counts[r0 + c0 + k] : 0;
      sum += v[k];
    }
    long long tot;
    long long ex = block_exclusive_scan(sum, &tot, lds) + carry;
#pragma unroll
    for (int k = 0; k < kScanPerThread; ++k) {
      if (c0 + k < ntiles) row_prefix[r0 + c0 + k] = static_cast<int32_t>(ex);
      ex += v[k];
    }
    carry += tot;
  }
  if (threadIdx.x == 0) row_total[blockIdx.x] = static_cast<int32_t>(carry);
}

// Static LDS of radix_scatter<BITS>. The host adds its size to the dynamic
// LDS of the interaction-backward workgroups a scatter launch carries, so the
// two must fit one workgroup's 160 KiB together.
template <int BITS>
struct ScatterLds {
  int wcount[kRadixWaves][1 << BITS];                        // per-wave running digit counts
  int gbase[1 << BITS];                                      // the tile's first output slot per digit
  int lds[kRadixWaves * ((1 << BITS) / kBwdThreads)];        // digit-total scan across the waves
};

// Stable scatter of one tile. Wave w owns keys [tile + w*512, +512) and walks
// them in rounds of 64 in their original order; equal digits inside a round
// are ranked by lane with ballots, and a per-wave running count per digit
// carries the rank across rounds. The tile's digit offsets come from the
// row-scanned count table (row_prefix, row_total) or, with row_prefix null,
// from the count table itself (at most kInlineScanTiles tiles).
template <int BITS>
__global__ __launch_bounds__(kBwdThreads) void radix_scatter(const int32_t* __restrict__ keys_in,
                                                             const int32_t* __restrict__ vals_in, long long n,
                                                             int shift, int ntiles,
                                                             const int32_t* __restrict__ counts,
                                                             const int32_t* __restrict__ row_prefix,
                                                             const int32_t* __restrict__ row_total,
                                                             int32_t* __restrict__ keys_out,
                                                             int32_t* __restrict__ vals_out,
                                                             const int32_t* __restrict__ bag_of,
                                                             int32_t* __restrict__ src_out, IbwdShare ia) {
  constexpr int kBins = 1 << BITS;
  if (ibwd_extra(ia, ntiles)) return;
  __shared__ ScatterLds<BITS> sm;
  auto& wcount = sm.wcount;
  int* gbase = sm.gbase;
  int* lds = sm.lds;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  for (int w = 0; w < kRadixWaves; ++w)
    for (int d = threadIdx.x; d < kBins; d += kBwdThreads) wcount[w][d] = 0;
  const long long sub = static_cast<long long>(blockIdx.x) * kRadixTile + static_cast<long long>(wave) * kRadixRounds * kWave;
  const unsigned long long lt = (1ull << lane) - 1ull;
  int key[kRadixRounds], val[kRadixRounds], dig[kRadixRounds], rank[kRadixRounds];
  // every round's key and value loads are issued first, so that they are in
  // flight while the tile's digit offsets are worked out
#pragma unroll
  for (int r = 0; r < kRadixRounds; ++r) {
    const long long i = sub + r * kWave + lane;
    key[r] = i < n ? keys_in[i] : 0;
    val[r] = i < n ? vals_in[i] : 0;
  }
  // last pass: the bag of each occurrence travels with it (src_out[dst] = bag_of[val])
  int src[kRadixRounds];
  if (src_out) {
#pragma unroll
    for (int r = 0; r < kRadixRounds; ++r) src[r] = bag_of[val[r]];  // val = 0 past the end: in bounds
  }
  tile_digit_base<BITS>(counts, row_prefix, row_total, ntiles, lds, gbase);
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kRadixRounds; ++r) {
    const long long i = sub + r * kWave + lane;
    const bool ok = i < n;
    const int d = (static_cast<uint32_t>(key[r]) >> shift) & (kBins - 1);
    dig[r] = ok ? d : -1;
    unsigned long long peers = __ballot(ok);
#pragma unroll
    for (int bit = 0; bit < BITS; ++bit) {
      const unsigned long long m = __ballot((d >> bit) & 1);
      peers &= ((d >> bit) & 1) ? m : ~m;
    }
    const int before = __popcll(peers & lt);
    const int cnt = __popcll(peers);
    int running = 0;
    if (ok) running = wcount[wave][d];
    __builtin_amdgcn_wave_barrier();
    if (ok && before == 0) wcount[wave][d] = running + cnt;
    __builtin_amdgcn_wave_barrier();
    rank[r] = running + before;
  }
  __syncthreads();
  for (int d = threadIdx.x; d < kBins; d += kBwdThreads) {
    int acc = 0;
    for (int w = 0; w < kRadixWaves; ++w) {
      const int c = wcount[w][d];
      wcount[w][d] = acc;
      acc += c;
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kRadixRounds; ++r) {
    if (dig[r] < 0) continue;
    const int dst = gbase[dig[r]] + wcount[wave][dig[r]] + rank[r];
    keys_out[dst] = key[r];
    vals_out[dst] = val[r];
    if (src_out) src_out[dst] = src[r];
  }
}

// ---------------------------------------------------------------------------
// 3b. per-table sort (small batches)
// ---------------------------------------------------------------------------
// Bags are in table-major order, so the occurrences of table t fill one range of
// positions [c_t, c_t+1), and every key of table t lies below every key of table
// t + 1. The stable order by key is therefore each table's stable order by row
// index, one table after another, followed by the occurrences with an
// out-of-range index and the positions outside every bag, in position order.
//  - table_sort: one workgroup per table sorts its range by row index (LSD, 8-bit
//    digits, as many passes as the table's row count needs; an out-of-range index
//    takes the key rows_t, so it sorts after the table's valid ones) and writes
//    it in that order to temporaries over the same range, with the table's count
//    of valid occurrences. A range of at most one tile (2048) stays in registers,
//    exchanged through LDS between passes; a longer one goes tile by tile through
//    the workspace.
//  - table_place: one workgroup per table moves its sorted range to the final
//    slots: its valid occurrences after those of the earlier tables, its invalid
//    ones after every valid occurrence, the gap positions and the invalid ones of
//    earlier tables. When every occurrence is valid, no position lies outside
//    the ranges and every range was sorted in registers, the final order is
//    each range in place, which table_sort has already written: table_place
//    then only checks that and returns.
// table_sort also carries the interaction-backward samples as extra workgroups.
// The table ranges are the offsets at the table boundaries, clamped into
// [0, nnz] and made non-decreasing (a running maximum), which changes nothing
// for a valid CSR.
constexpr int kTableTile = kRadixTile;  // occurrences a table sorts in registers: 8 per thread
constexpr int kTableBins = 1 << 8;

// table_sort's LDS (19 KiB), carved from the dynamic segment, which the
// interaction backward's extra workgroups of the same launch use for their own
// tile; the launch's dynamic LDS is the larger of the two.
struct TableSortLds {
  unsigned short wcount[kRadixWaves][kTableBins];  // per-wave digit counts, then their prefix over the waves
  int dbase[kTableBins];                           // first slot of each digit
  long long scan[kRadixWaves];                     // block scan across the waves
  int misc[4];                                     // [0] invalid occurrences
  union {
    struct {
      int xk[kTableTile];  // one-tile ranges: the keys and values between passes
      int xv[kTableTile];
    } x;
    struct {
      int hist[kTableBins];  // longer ranges: digit totals
      int cum[kTableBins];   // keys of each digit in the tiles done so far
    } m;
  };
};

struct TableSortArgs {
  int T, B;
  const int32_t* offsets;
  const int32_t* indices;
  long long nnz;
  int32_t* tkey;    // out [nnz]: each table's range sorted, its row index (rows_t for invalid)
  int32_t* tval;    // out [nnz]: ... and the occurrence's position
  int32_t* tbag;    // out [nnz]: ... and its bag's row of the pooled gradients (b * T + t)
  int32_t* tvalid;  // out [T]: valid occurrences per table
  int32_t* tbound;  // out [T + 1]: c_0 .. c_T
  // ranges longer than a tile: keys and values ping-pong between (k0, v0) and
  // (k1, v1); bag_of holds each position's bag
  int32_t* k0;
  int32_t* v0;
  int32_t* k1;
  int32_t* v1;
  int32_t* bag_of;  // as tbag, by position
  // a range of at most one tile also goes straight to the final arrays at its
  // own positions: the final order whenever every occurrence is valid and
  // every position lies in a range (table_place then leaves them as they are)
  int32_t* skeys;   // out [nnz]: global key, or the sentinel
  int32_t* src_bag; // out [nnz]: as tbag
  int32_t* perm;    // out [nnz] or null: the position
  int32_t sentinel;
  int32_t* status;
};

// c_t and c_t+1: the running maximum of the clamped table-boundary offsets,
// worked out by each wave on its own (a butterfly, no LDS, no barrier).
__device__ __forceinline__ void table_bounds(const int32_t* __restrict__ offsets, int B, long long nnz, int t,
                                             int& c0, int& c1) {
  const int lane = threadIdx.x & (kWave - 1);
  const int n = static_cast<int>(nnz);  // nnz < 2^31
  int m0 = 0, m1 = 0;
  for (int s = lane; s <= t + 1; s += kWave) {
    int o = offsets[static_cast<long long>(s) * B];
    o = o < 0 ? 0 : (o > n ? n : o);
    if (s <= t) m0 = o > m0 ? o : m0;
    m1 = o > m1 ? o : m1;
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const int y0 = __shfl_xor(m0, o, kWave), y1 = __shfl_xor(m1, o, kWave);
    m0 = y0 > m0 ? y0 : m0;
    m1 = y1 > m1 ? y1 : m1;
  }
  c0 = m0;
  c1 = m1;
}

// Stable ranking of one round of 64 keys of a wave by their digit d (ok false:
// no key): the number of equal digits at lower lanes, plus the wave's running
// count of that digit, which the round then advances.
__device__ __forceinline__ int rank_in_wave(int d, bool ok, unsigned short* wcnt) {
  unsigned long long peers = __ballot(ok);
#pragma unroll
  for (int bit = 0; bit < 8; ++bit) {
    const unsigned long long m = __ballot((d >> bit) & 1);
    peers &= ((d >> bit) & 1) ? m : ~m;
  }
  // set bits of peers at lower lanes
  const int before = static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<unsigned>(peers >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo(static_cast<unsigned>(peers), 0u)));
  const int cnt = __popcll(peers);
  int running = 0;
  if (ok) running = wcnt[d];
  __builtin_amdgcn_wave_barrier();
  if (ok && before == 0) wcnt[d] = static_cast<unsigned short>(running + cnt);
  __builtin_amdgcn_wave_barrier();
  return running + before;
}

// Thread d: turns the waves' counts of digit d into their exclusive prefix over
// the waves and returns the digit's total.
__device__ __forceinline__ int wave_prefix(TableSortLds& sm) {
  const int d = threadIdx.x;
  int tot = 0;
#pragma unroll
  for (int w = 0; w < kRadixWaves; ++w) {
    const int c = sm.wcount[w][d];
    sm.wcount[w][d] = static_cast<unsigned short>(tot);
    tot += c;
  }
  return tot;
}

__global__ __launch_bounds__(kBwdThreads) void table_sort(TableSortArgs a, MutTableArgs tabs, IbwdShare ia) {
  if (ibwd_extra(ia, a.T)) return;
  extern __shared__ __align__(16) float smem[];
  TableSortLds& sm = *reinterpret_cast<TableSortLds*>(smem);
  const int t = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int rows = tabs.rows[t];
  const long long bag0 = static_cast<long long>(t) * a.B;
  const long long nbags = static_cast<long long>(a.T) * a.B;
  // Bag j = (t, b) holds [o_j, max(o_j, o_j+1)) once clamped into [0, nnz] (the
  // CSR checks as in build_keys) and is recorded in bag_of, by position, as
  // b * T + t, its row of the pooled gradients. A position of the range that no
  // bag of this table holds (invalid offsets only) keeps the table's first bag, t.
  // The offsets of a thread's first kRadixRounds bags are loaded with the
  // table bounds, the indices right after: two memory round trips in all.
  constexpr int kBagBatch = kRadixRounds * kBwdThreads;
  int o0[kRadixRounds], o1[kRadixRounds];
#pragma unroll
  for (int u = 0; u < kRadixRounds; ++u) {
    const int j = threadIdx.x + u * kBwdThreads;
    const long long g = bag0 + (j < a.B ? j : 0);
    o0[u] = a.offsets[g];
    o1[u] = a.offsets[g + 1];
  }
  if (threadIdx.x == 0) sm.misc[0] = 0;
  int c0, c1;
  table_bounds(a.offsets, a.B, a.nnz, t, c0, c1);
  const int N = c1 - c0;
  const bool one_tile = N <= kTableTile;
  if (threadIdx.x == 0) {
    a.tbound[t] = c0;
    if (t == a.T - 1) a.tbound[a.T] = c1;
  }
  int idx[kRadixRounds];  // one-tile ranges: slot q = wave * 512 + r * 64 + lane holds position c0 + q
  if (one_tile) {
#pragma unroll
    for (int r = 0; r < kRadixRounds; ++r) {
      const int q = wave * kRadixRounds * kWave + r * kWave + lane;
      idx[r] = a.indices[q < N ? c0 + q : 0];
    }
  }
  for (int q = threadIdx.x; q < N; q += kBwdThreads) a.bag_of[c0 + q] = t;
  __syncthreads();  // the default bags are written
  bool bad_off = false;
  const int n = static_cast<int>(a.nnz);  // nnz < 2^31
  auto put_bag = [&](int j, int s0, int s1) {  // s0, s1: o_j, o_j+1
    const long long g = bag0 + j;
    if (g == 0 && s0 != 0) bad_off = true;
    if (g == nbags - 1 && s1 != n) bad_off = true;
    if (s0 < 0) { s0 = 0; bad_off = true; }
    if (s0 > n) { s0 = n; bad_off = true; }
    if (s1 < 0) { s1 = 0; bad_off = true; }
    if (s1 > n) { s1 = n; bad_off = true; }
    if (s1 < s0) { s1 = s0; bad_off = true; }
    const int p0 = s0 > c0 ? s0 : c0, p1 = s1 < c1 ? s1 : c1;
    const int row = j * a.T + t;
    for (int p = p0; p < p1; ++p) a.bag_of[p] = row;
  };
#pragma unroll
  for (int u = 0; u < kRadixRounds; ++u) {
    const int j = threadIdx.x + u * kBwdThreads;
    if (j < a.B) put_bag(j, o0[u], o1[u]);
  }
  for (int j = threadIdx.x + kBagBatch; j < a.B; j += kBwdThreads) put_bag(j, a.offsets[bag0 + j], a.offsets[bag0 + j + 1]);
  if (bad_off) flag(a.status, DLRM_STATUS_BAD_OFFSETS);
  // keys are in [0, rows]: as many 8-bit passes as rows needs bits
  const int passes = (32 - __clz(rows) + 7) / 8;
  int nbad = 0;
  if (one_tile) {
    // keys in registers
    int key[kRadixRounds], val[kRadixRounds];
#pragma unroll
    for (int r = 0; r < kRadixRounds; ++r) {
      const int q = wave * kRadixRounds * kWave + r * kWave + lane;
      const bool ok = q < N;
      const bool valid = idx[r] >= 0 && idx[r] < rows;
      key[r] = valid ? idx[r] : rows;
      val[r] = q;  // the occurrence's slot (its position less c0)
      nbad += (ok && !valid) ? 1 : 0;
    }
    // the passes: rank in each wave, prefix over the waves and digits, exchange;
    // a slot and its rank (both below 2^16) share a register until the exchange
    for (int ps = 0; ps < passes; ++ps) {
      const int shift = 8 * ps;
#pragma unroll
      for (int w = 0; w < kRadixWaves; ++w) sm.wcount[w][threadIdx.x] = 0;
      __syncthreads();
#pragma unroll
      for (int r = 0; r < kRadixRounds; ++r) {
        const int q = wave * kRadixRounds * kWave + r * kWave + lane;
        const int d = (key[r] >> shift) & (kTableBins - 1);
        val[r] = (val[r] << 16) | rank_in_wave(d, q < N, sm.wcount[wave]);
      }
      __syncthreads();
      long long total;
      const int tot = wave_prefix(sm);
      sm.dbase[threadIdx.x] = static_cast<int>(block_exclusive_scan(tot, &total, sm.scan));
      __syncthreads();
#pragma unroll
      for (int r = 0; r < kRadixRounds; ++r) {
        const int q = wave * kRadixRounds * kWave + r * kWave + lane;
        if (q >= N) continue;
        const int d = (key[r] >> shift) & (kTableBins - 1);
        const int dst = sm.dbase[d] + sm.wcount[wave][d] + (val[r] & 0xffff);
        sm.x.xk[dst] = key[r];
        sm.x.xv[dst] = val[r] >> 16;
      }
      __syncthreads();
#pragma unroll
      for (int r = 0; r < kRadixRounds; ++r) {
        const int q = wave * kRadixRounds * kWave + r * kWave + lane;
        if (q < N) {
          key[r] = sm.x.xk[q];
          val[r] = sm.x.xv[q];
        }
      }
    }
    // the sorted range, with each occurrence's bag (the bags were stored before
    // at least one barrier: every pass, and the one below with no pass, has one)
    if (passes == 0) __syncthreads();
#pragma unroll
    for (int r = 0; r < kRadixRounds; ++r) {
      const int q = wave * kRadixRounds * kWave + r * kWave + lane;
      if (q < N) {
        const int bag = a.bag_of[c0 + val[r]];
        a.tkey[c0 + q] = key[r];
        a.tval[c0 + q] = c0 + val[r];
        a.tbag[c0 + q] = bag;
        a.skeys[c0 + q] = key[r] < rows ? tabs.base[t] + key[r] : a.sentinel;
        a.src_bag[c0 + q] = bag;
        if (a.perm) a.perm[c0 + q] = c0 + val[r];
      }
    }
  } else {
    __syncthreads();  // the bags are in the workspace
    // keys through the workspace
    for (int q = threadIdx.x; q < N; q += kBwdThreads) {
      const int ix = a.indices[c0 + q];
      const bool valid = ix >= 0 && ix < rows;
      a.k0[c0 + q] = valid ? ix : rows;
      a.v0[c0 + q] = c0 + q;
      nbad += valid ? 0 : 1;
    }
    __syncthreads();
    const int32_t* sk = a.k0;
    const int32_t* sv = a.v0;
    if (passes == 0) {  // a single row: the order stays the positions'
      for (int q = threadIdx.x; q < N; q += kBwdThreads) {
        a.tkey[c0 + q] = sk[c0 + q];
        a.tval[c0 + q] = sv[c0 + q];
        a.tbag[c0 + q] = a.bag_of[sv[c0 + q]];
      }
    }
    for (int ps = 0; ps < passes; ++ps) {
      const int shift = 8 * ps;
      const bool last = ps + 1 == passes;
      int32_t* dk = last ? a.tkey : ((ps & 1) ? a.k0 : a.k1);
      int32_t* dv = last ? a.tval : ((ps & 1) ? a.v0 : a.v1);
      // digit totals over the whole range, then their exclusive scan
      sm.m.hist[threadIdx.x] = 0;
      __syncthreads();
      for (int q = threadIdx.x; q < N; q += kBwdThreads) atomicAdd(&sm.m.hist[(sk[c0 + q] >> shift) & (kTableBins - 1)], 1);
      __syncthreads();
      long long total;
      sm.dbase[threadIdx.x] = static_cast<int>(block_exclusive_scan(sm.m.hist[threadIdx.x], &total, sm.scan));
      sm.m.cum[threadIdx.x] = 0;
      // tiles in position order, each ranked like a one-tile range
      for (int q0 = 0; q0 < N; q0 += kTableTile) {
#pragma unroll
        for (int w = 0; w < kRadixWaves; ++w) sm.wcount[w][threadIdx.x] = 0;
        __syncthreads();
        int key[kRadixRounds], val[kRadixRounds], rank[kRadixRounds];
#pragma unroll
        for (int r = 0; r < kRadixRounds; ++r) {
          const int q = q0 + wave * kRadixRounds * kWave + r * kWave + lane;
          const bool ok = q < N;
          key[r] = ok ? sk[c0 + q] : 0;
          val[r] = ok ? sv[c0 + q] : 0;
          rank[r] = rank_in_wave((key[r] >> shift) & (kTableBins - 1), ok, sm.wcount[wave]);
        }
        __syncthreads();
        sm.m.hist[threadIdx.x] = wave_prefix(sm);  // this tile's digit totals
        __syncthreads();
#pragma unroll
        for (int r = 0; r < kRadixRounds; ++r) {
          if (q0 + wave * kRadixRounds * kWave + r * kWave + lane >= N) continue;
          const int d = (key[r] >> shift) & (kTableBins - 1);
          const int dst = c0 + sm.dbase[d] + sm.m.cum[d] + sm.wcount[wave][d] + rank[r];
          dk[dst] = key[r];
          dv[dst] = val[r];
          if (last) a.tbag[dst] = a.bag_of[val[r]];
        }
        __syncthreads();
        sm.m.cum[threadIdx.x] += sm.m.hist[threadIdx.x];
      }
      __syncthreads();  // this pass's output is the next one's input
      sk = dk;
      sv = dv;
    }
  }
  // valid occurrences of the table
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) nbad += __shfl_xor(nbad, o, kWave);
  if (lane == 0 && nbad) atomicAdd(&sm.misc[0], nbad);
  __syncthreads();
  if (threadIdx.x == 0) {
    a.tvalid[t] = N - sm.misc[0];
    if (sm.misc[0]) flag(a.status, DLRM_STATUS_BAD_INDEX);
  }
}

// The final order (see table_sort): sorted keys, the permutation (if wanted) and
// each sorted position's bag.
__global__ __launch_bounds__(kBwdThreads) void table_place(const int32_t* __restrict__ tkey,
                                                           const int32_t* __restrict__ tval,
                                                           const int32_t* __restrict__ tbag,
                                                           const int32_t* __restrict__ tvalid,
                                                           const int32_t* __restrict__ tbound, MutTableArgs tabs,
                                                           int T, long long nnz, int32_t sentinel,
                                                           int32_t* __restrict__ skeys, int32_t* __restrict__ perm,
                                                           int32_t* __restrict__ src_bag) {
  __shared__ int red[2][kRadixWaves];
  const int t = blockIdx.x;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const int c0 = tbound[t], c1 = tbound[t + 1], nvalid = tvalid[t];
  // valid occurrences of the tables before t (before) and of all tables (all)
  int before = 0, all = 0;
  for (int s = threadIdx.x; s < T; s += kBwdThreads) {
    const int v = tvalid[s];
    all += v;
    before += s < t ? v : 0;
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    before += __shfl_xor(before, o, kWave);
    all += __shfl_xor(all, o, kWave);
  }
  if (lane == 0) {
    red[0][wave] = before;
    red[1][wave] = all;
  }
  __syncthreads();
  before = 0;
  all = 0;
#pragma unroll
  for (int w = 0; w < kRadixWaves; ++w) {
    before += red[0][w];
    all += red[1][w];
  }
  // every position valid and in a range (all = nnz), and every range sorted in
  // registers: table_sort has already written the final order
  bool longer = false;
  for (int s = threadIdx.x; s < T; s += kBwdThreads) longer |= tbound[s + 1] - tbound[s] > kTableTile;
  __syncthreads();  // red is read by every thread above before it is reused
  const unsigned long long any_longer = __ballot(longer);  // every lane votes (not in lane 0's branch)
  if (lane == 0) red[0][wave] = any_longer != 0ull;
  __syncthreads();
  longer = false;
#pragma unroll
  for (int w = 0; w < kRadixWaves; ++w) longer |= red[0][w] != 0;
  if (all == nnz && !longer) return;
  const int base = tabs.base[t];
  // the invalid occurrences before this table's: the gap in front (c_0 positions)
  // and those of the earlier tables (c_t - c_0 - before)
  const int bad_first = all + c0 - before;
  // kRadixRounds entries per thread in flight: all loads of a batch before its stores
  for (int s0 = 0; s0 < c1 - c0; s0 += kRadixRounds * kBwdThreads) {
    int k[kRadixRounds], v[kRadixRounds], g[kRadixRounds];
#pragma unroll
    for (int u = 0; u < kRadixRounds; ++u) {
      const int s = s0 + u * kBwdThreads + threadIdx.x;
      const int q = s < c1 - c0 ? c0 + s : c0;
      k[u] = tkey[q];
      v[u] = tval[q];
      g[u] = tbag[q];
    }
#pragma unroll
    for (int u = 0; u < kRadixRounds; ++u) {
      const int s = s0 + u * kBwdThreads + threadIdx.x;
      if (s < c1 - c0) {
        const bool ok = s < nvalid;
        const int out = ok ? before + s : bad_first + (s - nvalid);
        skeys[out] = ok ? base + k[u] : sentinel;
        if (perm) perm[out] = v[u];
        src_bag[out] = g[u];
      }
    }
  }
  // positions outside every table's range (invalid offsets only): in front of c_0,
  // and from c_T on (which stay where they are)
  if (t == 0) {
    for (int p = threadIdx.x; p < tbound[0]; p += kBwdThreads) {
      skeys[all + p] = sentinel;
      if (perm) perm[all + p] = p;
      src_bag[all + p] = 0;
    }
  }
  if (t == T - 1) {
    for (long long p = tbound[T] + threadIdx.x; p < nnz; p += kBwdThreads) {
      skeys[p] = sentinel;
      if (perm) perm[p] = static_cast<int32_t>(p);
      src_bag[p] = 0;
    }
  }
}

struct HeadIn {
  const int32_t* keys;
  int32_t sentinel;
  __device__ __forceinline__ long long operator()(long long i) const {
    const int32_t k = keys[i];
    return (k != sentinel && (i == 0 || keys[i - 1] != k)) ? 1 : 0;
  }
};

// ---------------------------------------------------------------------------
// 4. segments
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBwdThreads) void build_segments(const int32_t* __restrict__ keys, long long n,
                                                              int32_t sentinel, const int32_t* __restrict__ pos,
                                                              int32_t* __restrict__ unique_keys,
                                                              int32_t* __restrict__ seg_offsets,
                                                              int32_t* __restrict__ num_unique) {
  const long long i = static_cast<long long>(blockIdx.x) * kBwdThreads + threadIdx.x;
  if (i >= n) return;
  const int32_t k = keys[i];
  const bool valid = k != sentinel;
  if (valid && (i == 0 || keys[i - 1] != k)) {
    unique_keys[pos[i]] = k;
    seg_offsets[pos[i]] = static_cast<int32_t>(i);
  }
  // the last valid key closes the segment list
  const bool last_valid = valid && (i + 1 == n || keys[i + 1] == sentinel);
  const bool none_valid = i == 0 && !valid;
  if (last_valid || none_valid) {
    const int32_t U = pos[n];
    seg_offsets[U] = last_valid ? static_cast<int32_t>(i + 1) : 0;
    *num_unique = U;
  }
}

// Static LDS of build_segments_chunked (see ScatterLds).
struct SegChunkedLds {
  long long lds[kScanThreads / kWave];
};

// The same for up to 256 scan chunks, in one pass after the chunk totals:
// each workgroup adds up the totals of the chunks before its own, scans its
// chunk's head flags, and writes pos (pos[i] = heads before position i, pos[n]
// = all heads), the segment starts and keys, and the segment count.
__global__ __launch_bounds__(kScanThreads) void build_segments_chunked(const int32_t* __restrict__ keys, long long n,
                                                                      int32_t sentinel,
                                                                      const long long* __restrict__ partial,
                                                                      int32_t* __restrict__ pos,
                                                                      int32_t* __restrict__ unique_keys,
                                                                      int32_t* __restrict__ seg_offsets,
                                                                      int32_t* __restrict__ num_unique, int nchunks,
                                                                      IbwdShare ia) {
  static_assert(kScanThreads == kBwdThreads, "extra workgroups run the interaction backward");
  if (ibwd_extra(ia, nchunks)) return;
  __shared__ SegChunkedLds sm;
  long long* lds = sm.lds;
  const long long c0 = static_cast<long long>(blockIdx.x) * kScanChunk + threadIdx.x * kScanPerThread;
  // totals of the earlier chunks (at most 256, one per thread)
  const long long pv = threadIdx.x < blockIdx.x ? partial[threadIdx.x] : 0;
  int32_t k[kScanPerThread + 2];  // k[j] = key c0 - 1 + j, for c0 - 1 .. c0 + 16 (outside [0, n): the sentinel)
#pragma unroll
  for (int j = 0; j < kScanPerThread + 2; ++j) {
    const long long i = c0 - 1 + j;
    k[j] = (i >= 0 && i < n) ? keys[i] : sentinel;
  }
  long long tot_before;
  block_exclusive_scan(pv, &tot_before, lds);
  int h[kScanPerThread];
  long long s = 0;
#pragma unroll
  for (int j = 0; j < kScanPerThread; ++j) {
    const int32_t kk = k[j + 1];
    h[j] = (c0 + j < n && kk != sentinel && (c0 + j == 0 || k[j] != kk)) ? 1 : 0;
    s += h[j];
  }
  long long chunk_tot;
  long long ex = block_exclusive_scan(s, &chunk_tot, lds) + tot_before;
#pragma unroll
  for (int j = 0; j < kScanPerThread; ++j) {
    const long long i = c0 + j;
    if (i < n) {
      pos[i] = static_cast<int32_t>(ex);
      if (h[j]) {
        unique_keys[ex] = k[j + 1];
        seg_offsets[ex] = static_cast<int32_t>(i);
      }
      // the last valid key closes the segment list
      const bool valid = k[j + 1] != sentinel;
      const bool last_valid = valid && (i + 1 == n || k[j + 2] == sentinel);
      const bool none_valid = i == 0 && !valid;
      if (last_valid || none_valid) {
        const long long U = ex + h[j];
        seg_offsets[U] = last_valid ? static_cast<int32_t>(i + 1) : 0;
        *num_unique = static_cast<int32_t>(U);
      }
    }
    ex += h[j];
  }
  if (static_cast<int>(blockIdx.x) == nchunks - 1 && threadIdx.x == 0) pos[n] = static_cast<int32_t>(tot_before + chunk_tot);
}

__global__ void zero_segments(int32_t* seg_offsets, int32_t* num_unique) {
  if (threadIdx.x == 0) {
    seg_offsets[0] = 0;
    *num_unique = 0;
  }
}


// ---------------------------------------------------------------------------
// 5. segmented reduce + SGD over fixed chunks of the sorted occurrences
// ---------------------------------------------------------------------------
// The sorted occurrences are cut into chunks of C consecutive positions, one
// wave each, whatever the segment lengths (a Zipf-hot row can own thousands of
// occurrences). A wave loads the C gradient rows of its chunk at once, then
// sums them in position order, closing a sum at every segment end:
//   - a segment that starts and ends in the chunk gets its SGD update here;
//   - the part of a segment that began in an earlier chunk goes to carry[k];
//   - the first part of a segment that goes on past the chunk goes to head[k].
// seg_combine then adds head[k] + carry[k+1] + ... in chunk order for every
// segment that crosses a chunk end and applies its update. The summation
// order depends only on the positions, so results are deterministic.
//
// Row layout in registers: lane l holds EL fp32 columns [c, c + EL) of a
// d_pooled row, c = (l % LPR) * EL, LPR = min(64, D) lanes per row (for D < 64
// the lanes above D repeat lanes 0..D-1 and write the same values).
constexpr int kChunkFirstCont = 1;  // the chunk's first segment began in an earlier chunk
constexpr int kChunkLastCont = 2;   // the chunk's last segment goes on into the next chunk
constexpr int kChunkSingle = 4;     // the chunk holds (part of) one segment only

template <int EL>
struct RowVec {
  float v[EL];
  __device__ __forceinline__ void load(const float* p) {
    if constexpr (EL == 1) v[0] = *p;
    else if constexpr (EL == 2) { const float2 x = *reinterpret_cast<const float2*>(p); v[0] = x.x; v[1] = x.y; }
    else {
#pragma unroll
      for (int i = 0; i < EL; i += 4) {
        const float4 x = *reinterpret_cast<const float4*>(p + i);
        v[i] = x.x; v[i + 1] = x.y; v[i + 2] = x.z; v[i + 3] = x.w;
      }
    }
  }
  __device__ __forceinline__ void store(float* p) const {
    if constexpr (EL == 1) *p = v[0];
    else if constexpr (EL == 2) *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
    else {
#pragma unroll
      for (int i = 0; i < EL; i += 4) *reinterpret_cast<float4*>(p + i) = make_float4(v[i], v[i + 1], v[i + 2], v[i + 3]);
    }
  }
};

// Table row of a global key: table t (the last whose base is <= key) and the
// row's first element.
struct RowRef {
  int t;
  size_t off;
};

__device__ __forceinline__ RowRef row_of_key(const MutTableArgs& tabs, int T, int D, int key) {
  int t = 0;  // bases ascend
#pragma unroll
  for (int step = 64; step > 0; step >>= 1) {
    const int c = t + step;
    if (c < T && tabs.base[c] <= key) t = c;
  }
  return RowRef{t, static_cast<size_t>(key - tabs.base[t]) * D};
}

// This lane's EL columns of a table row, widened to fp32 (exactly), and the
// SGD write-back W - lr * g, rounded once to the storage type.
template <int DT, int EL>
struct TabVec {
  float v[EL];
  __device__ __forceinline__ void load(const MutTableArgs& tabs, RowRef r, int col) {
    if constexpr (DT == DLRM_F32) {
      RowVec<EL> x;
      x.load(static_cast<const float*>(tabs.ptr[r.t]) + r.off + col);
#pragma unroll
      for (int e = 0; e < EL; ++e) v[e] = x.v[e];
    } else {
      const uint16_t* w = static_cast<const uint16_t*>(tabs.ptr[r.t]) + r.off + col;
#pragma unroll
      for (int e = 0; e < EL; ++e) {
        const uint32_t bits = w[e];
        v[e] = DT == DLRM_BF16 ? bf16_lo(bits) : f16_lo(bits);
      }
    }
  }
  // W - step * g with step = lr (SGD) or lr / (sqrt(state) + eps) (row-wise AdaGrad)
  __device__ __forceinline__ void sgd_store(const MutTableArgs& tabs, RowRef r, int col, const RowVec<EL>& g,
                                            float lr) const {
    const float nlr = -lr;
    if constexpr (DT == DLRM_F32) {
      RowVec<EL> x;
#pragma unroll
      for (int e = 0; e < EL; ++e) x.v[e] = fmaf(nlr, g.v[e], v[e]);
      x.store(static_cast<float*>(tabs.ptr[r.t]) + r.off + col);
    } else {
      uint16_t* w = static_cast<uint16_t*>(tabs.ptr[r.t]) + r.off + col;
#pragma unroll
      for (int e = 0; e < EL; ++e) w[e] = to_half_bits<DT>(fmaf(nlr, g.v[e], v[e]));
    }
  }
};

// Row-wise AdaGrad on a segment's summed gradient g (this lane's EL columns):
// state <- state + mean over the row of g^2, then step = lr / (sqrt(state) + eps).
// The sum of squares is a butterfly over the wave (fixed order); lanes that
// repeat columns (D < 64) contribute nothing. Lane 0 writes the new state.
template <int EL>
__device__ __forceinline__ float adagrad_step(const RowVec<EL>& g, float s_old, float* s_ptr, int D, float lr,
                                              float eps) {
  const int lane = threadIdx.x & (kWave - 1);
  const int lpr = D < kWave ? D : kWave;
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < EL; ++e) ss = fmaf(g.v[e], g.v[e], ss);
  if (lane >= lpr) ss = 0.f;
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) ss += shfl_xor_f(ss, m);
  const float s_new = s_old + ss / static_cast<float>(D);
  if (lane == 0) *s_ptr = s_new;
  return lr / (sqrtf(s_new) + eps);
}

template <int DT, int EL, int C, int OPT>
__global__ __launch_bounds__(kBwdThreads) void seg_reduce_chunks(MutTableArgs tabs, StateArgs state, float eps, int T, int D,
                                                                 const int32_t* __restrict__ skeys, long long n,
                                                                 int32_t sentinel,
                                                                 const int32_t* __restrict__ src_bag,
                                                                 const float* __restrict__ d_pooled, int nbags, float lr,
                                                                 float* __restrict__ carry, float* __restrict__ head,
                                                                 float* __restrict__ wgcarry,
                                                                 int32_t* __restrict__ chunk_flags, long long nchunks,
                                                                 int32_t* __restrict__ hcount, int32_t* __restrict__ hwg) {
  static_assert(C <= kWave, "one lane per chunk position");
  constexpr int kWaves = kBwdThreads / kWave;
  __shared__ int sbase[DLRM_MAX_TABLES];  // first global key of each table
  __shared__ float* sstate[OPT == kRowwiseAdagrad ? DLRM_MAX_TABLES : 1];  // each table's row states
  __shared__ int wg_heads, wg_done, wg_pure;  // the workgroup's heads so far, its waves done, its pure chunks
  __shared__ float wcarry[kWaves][kWave * EL];  // the carries of pure chunks
  for (int t = threadIdx.x; t < T; t += kBwdThreads) {
    sbase[t] = tabs.base[t];
    if constexpr (OPT == kRowwiseAdagrad) sstate[t] = state.ptr[t];
  }
  if (threadIdx.x == 0) {
    wg_heads = 0;
    wg_done = 0;
    wg_pure = 0;
  }
  __syncthreads();
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  const int lpr = D < kWave ? D : kWave;
  const int col = (lane % lpr) * EL;
  // Each XCD takes a contiguous run of chunks (the workgroups it is dealt are
  // renumbered): the sorted occurrences of a run belong to one or a few
  // tables, so the pooled-gradient rows its chunks gather (one bag row is read
  // once per occurrence in the bag) come from a slice that fits its L2.
  const int wg = xcd_block(blockIdx.x, gridDim.x);
  // Every wave ends here with its chunk's number of segment starts (heads):
  // it adds them to the workgroup's sum, then counts itself done; the last of
  // the four stores the sum for the combine step's prefix sums (no barrier, so
  // waves may leave early). When all four chunks are pure (wholly inside one
  // segment that began before them and goes on after them), the last wave also
  // stores the sum of their four carries, in wave order, as the workgroup's
  // carry: the combine step then adds a long segment's carries four chunks at
  // a time.
  auto finish = [&](int heads) {
    int last = 0;
    if (lane == 0) {
      if (hwg) atomicAdd(&wg_heads, heads);
      __threadfence_block();
      last = atomicAdd(&wg_done, 1) == kWaves - 1;
    }
    if (__builtin_amdgcn_readfirstlane(last)) {
      __threadfence_block();
      if (hwg && lane == 0) hwg[wg] = atomicAdd(&wg_heads, 0);
      if (atomicAdd(&wg_pure, 0) == kWaves) {
#pragma unroll
        for (int e = 0; e < EL; ++e) {
          float v = wcarry[0][col + e];
#pragma unroll
          for (int w = 1; w < kWaves; ++w) v += wcarry[w][col + e];
          wgcarry[static_cast<size_t>(wg) * D + col + e] = v;
        }
      }
    }
  };
  const long long k = static_cast<long long>(wg) * (kBwdThreads / kWave) + (threadIdx.x >> 6);
  if (k >= nchunks) {
    finish(0);
    return;
  }
  const long long q0 = k * C;
  // per position (lane j < C): its key (sorted), the key before it, the key
  // after it, and the bag whose gradient row it adds; all independent loads.
  // Valid keys form a prefix (the sentinel sorts last). Slots past the chunk
  // or past the valid keys repeat the chunk's first position.
  const long long qa = q0 + lane;
  const bool in_n = lane < C && qa < n;
  const long long qc = in_n ? qa : q0;
  const int key_raw = skeys[qc];
  const int key_prev = qc > 0 ? skeys[qc - 1] : -1;
  const int key_next = qc + 1 < n ? skeys[qc + 1] : sentinel;
  const int src_raw = src_bag[qc];
  const unsigned long long valid_mask = __ballot(in_n && key_raw != sentinel);
  const int nq = __popcll(valid_mask);
  if (nq == 0) {
    if (lane == 0) {
      chunk_flags[k] = 0;
      if (hcount) hcount[k] = 0;
    }
    finish(0);
    return;
  }
  const bool mine = lane < nq;
  const int key = mine ? key_raw : __shfl(key_raw, 0, kWave);
  // a bag row outside [0, B*T) would be an error of an earlier step; it is
  // clamped so that the gradient reads stay inside d_pooled whatever happens
  int src = mine ? src_raw : __shfl(src_raw, 0, kWave);
  src = src < 0 ? 0 : (src >= nbags ? nbags - 1 : src);
  // the position after the chunk's last valid one starts a new segment, or is
  // the end of the valid keys
  const int last_next = __shfl(key_next, nq - 1, kWave);
  const bool next_starts = nq < C || last_next == sentinel || last_next != __shfl(key_raw, nq - 1, kWave);
  int tk = 0;  // table of this lane's key: the last one whose base is <= key
#pragma unroll
  for (int step = 64; step > 0; step >>= 1) {
    const int c = tk + step;
    const int b = sbase[c < T ? c : T - 1];
    if (c < T && b <= key) tk = c;
  }
  const int rk = key - sbase[tk];
  // row-wise AdaGrad: the state of this lane's row, one gather for the wave
  // (lanes past the valid keys repeat lane 0's row: in bounds)
  float s_lane = 0.f;
  if constexpr (OPT == kRowwiseAdagrad) s_lane = sstate[tk][rk];
  const bool starts = mine && (qa == 0 || key_prev != key_raw);
  // does a segment start right after the chunk? (then the last one closes here)
  const unsigned long long start_mask = __ballot(starts);
  const unsigned long long lane_bit = 1ull << lane;
  // position j closes a segment if a segment starts at j + 1 or j is the last one
  const bool closes = lane < nq && (lane + 1 == nq || ((start_mask >> (lane + 1)) & 1ull));
  const bool first_cont = !(start_mask & 1ull);
  // a closing segment began before the chunk if no segment starts in (0, j]
  const bool began_before = first_cont && (start_mask & (lane_bit | (lane_bit - 1)) & ~1ull) == 0;
  const bool goes_on = lane + 1 == nq && !next_starts;
  const unsigned long long complete_mask = __ballot(closes && !began_before && !goes_on);
  const unsigned long long carry_mask = __ballot(closes && began_before);
  int flags = first_cont ? kChunkFirstCont : 0;
  if (!next_starts) flags |= kChunkLastCont;
  if (__popcll(start_mask) + (first_cont ? 1 : 0) == 1) flags |= kChunkSingle;
  const bool pure = flags == (kChunkFirstCont | kChunkLastCont | kChunkSingle);

  // all gradient rows and the table rows of the segments completed here are
  // loaded up front (slots without a completed segment re-read its first row)
  // A slot's table row is named by its lane's (tk, rk), read into scalars where
  // the row is loaded and again where it is stored, rather than kept in 32
  // scalar registers per slot in between (which spilled).
  auto ref_of = [&](int j) {
    return RowRef{__builtin_amdgcn_readlane(tk, j),
                  static_cast<size_t>(__builtin_amdgcn_readlane(rk, j)) * static_cast<size_t>(D)};
  };
  RowVec<EL> rows[C];
  TabVec<DT, EL> trow[C];
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int r = __shfl(src, j, kWave);
    rows[j].load(d_pooled + static_cast<size_t>(r) * D + col);
    const int jj = ((complete_mask >> j) & 1ull) ? j : 0;
    trow[j].load(tabs, ref_of(jj), col);
  }
  RowVec<EL> acc;
#pragma unroll
  for (int e = 0; e < EL; ++e) acc.v[e] = 0.f;
  const unsigned long long close_mask = __ballot(closes);
#pragma unroll
  for (int j = 0; j < C; ++j) {
    if (j < nq) {
#pragma unroll
      for (int e = 0; e < EL; ++e) acc.v[e] += rows[j].v[e];
      if ((close_mask >> j) & 1ull) {
        if ((complete_mask >> j) & 1ull) {
          const RowRef ref = ref_of(j);
          if constexpr (OPT == kRowwiseAdagrad) {
            // a complete segment closes at j, so lane j holds its row and that row's state
            const int rj = __builtin_amdgcn_readlane(rk, j);
            const float s_old = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s_lane), j));
            trow[j].sgd_store(tabs, ref, col, acc, adagrad_step<EL>(acc, s_old, sstate[ref.t] + rj, D, lr, eps));
          } else {
            trow[j].sgd_store(tabs, ref, col, acc, lr);
          }
        } else if ((carry_mask >> j) & 1ull) {
          // the chunk's first segment, begun in an earlier chunk, ends or runs through here
          acc.store(carry + static_cast<size_t>(k) * D + col);
          if (pure) {
#pragma unroll
            for (int e = 0; e < EL; ++e) wcarry[wave][col + e] = acc.v[e];
          }
        } else {
          // a segment begun here that goes on into the next chunk
          acc.store(head + static_cast<size_t>(k) * D + col);
        }
#pragma unroll
        for (int e = 0; e < EL; ++e) acc.v[e] = 0.f;
      }
    }
  }
  if (lane == 0) {
    chunk_flags[k] = flags;
    if (hcount) hcount[k] = __popcll(start_mask);  // the chunk's segment starts (heads)
    if (pure) {
      __threadfence_block();  // the wave's carry is in LDS
      atomicAdd(&wg_pure, 1);
    }
  }
  finish(__popcll(start_mask));
}

// Segment outputs written by seg_combine from the reduce's per-chunk head
// counts (hcount null: not built there).
struct SegOut {
  int32_t* hcount;  // per chunk: written by the reduce, read by the combine step
  int32_t* hwg;     // per reduce workgroup of four chunks: the same, summed
  int32_t* unique_keys;
  int32_t* seg_offsets;
  int32_t* num_unique;
  long long n;
  int32_t sentinel;
};

// Up to this many reduce chunks, seg_combine writes the segment outputs: each
// workgroup sums the head totals of all workgroups before its own (up to 8
// 16-byte loads per thread, from L2), so the total reads grow with the square
// of the count (about 130 MB at the limit).
constexpr long long kFusedSegChunks = 32768;

// The segment outputs of this workgroup's chunks (one per wave): a head is a
// valid key that differs from its predecessor; its index among all heads is
// the heads of the earlier chunks plus its rank in the chunk. The wave holding
// the last valid key (or position 0 when there is none) closes the list.
template <int C>
__device__ __forceinline__ void write_segments(const SegOut& so, const int32_t* __restrict__ skeys, long long nchunks) {
  constexpr int kW = kBwdThreads / kWave;  // chunks per workgroup (the reduce's and this launch's)
  __shared__ int red[kW], own[kW];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
  const long long w0 = static_cast<long long>(blockIdx.x) * kW;
  // this wave's keys first (a wave past the last chunk reads the last chunk's
  // and writes nothing), so that their loads and the prefix loads below share
  // one round trip
  const long long k = w0 + wave;
  const long long kc = k < nchunks ? k : nchunks - 1;
  const long long q = kc * C + lane;
  const bool in = k < nchunks && lane < C && q < so.n;
  const long long qc = lane < C && q < so.n ? q : kc * C;  // kc * C < n for every chunk
  const int32_t key = skeys[qc];
  const int32_t prev = qc > 0 ? skeys[qc - 1] : so.sentinel;
  const int32_t next = qc + 1 < so.n ? skeys[qc + 1] : so.sentinel;
  // heads of the chunks before this workgroup's: the totals of the earlier
  // workgroups, read 4 at a time (hwg is 16-byte aligned), so that up to 8192
  // of them take one round of loads
  const int nbefore = static_cast<int>(blockIdx.x);
  const int n4 = nbefore >> 2;
  const int4* h4 = reinterpret_cast<const int4*>(so.hwg);
  int sum = 0;
  for (int i0 = threadIdx.x; i0 < n4; i0 += 8 * kBwdThreads) {
    int4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * kBwdThreads;
      v[u] = i < n4 ? h4[i] : make_int4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) sum += v[u].x + v[u].y + v[u].z + v[u].w;
  }
  if (4 * n4 + static_cast<int>(threadIdx.x) < nbefore) sum += so.hwg[4 * n4 + threadIdx.x];  // the last 0..3
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) sum += __shfl_xor(sum, m, kWave);
  if (lane == 0) {
    red[wave] = sum;
    own[wave] = w0 + wave < nchunks ? so.hcount[w0 + wave] : 0;
  }
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int w = 0; w < kW; ++w) before += red[w] + (w < wave ? own[w] : 0);
  if (k >= nchunks) return;
  const bool valid = in && key != so.sentinel;
  const bool is_head = valid && (q == 0 || prev != key);
  const unsigned long long hm = __ballot(is_head);
  const int idx = before + __popcll(hm & ((1ull << lane) - 1ull));
  if (is_head) {
    so.unique_keys[idx] = key;
    so.seg_offsets[idx] = static_cast<int32_t>(q);
  }
  const bool last_valid = valid && (q + 1 == so.n || next == so.sentinel);
  const bool none_valid = in && q == 0 && !valid;
  if (last_valid || none_valid) {
    const int U = before + __popcll(hm);  // no head lies past the last valid key
    so.seg_offsets[U] = last_valid ? static_cast<int32_t>(q + 1) : 0;
    *so.num_unique = U;
  }
}

// The update of one segment's row (this lane's EL columns).
template <int DT, int EL, int OPT>
__device__ __forceinline__ void row_update(const MutTableArgs& tabs, const StateArgs& state, float eps, int T, int D,
                                           int key, int col, const RowVec<EL>& g, float lr) {
  const RowRef r = row_of_key(tabs, T, D, key);
  TabVec<DT, EL> x;
  x.load(tabs, r, col);
  if constexpr (OPT == kRowwiseAdagrad) {
    const int row = key - tabs.base[r.t];
    x.sgd_store(tabs, r, col, g, adagrad_step<EL>(g, state.ptr[r.t][row], state.ptr[r.t] + row, D, lr, eps));
  } else {
    x.sgd_store(tabs, r, col, g, lr);
  }
}

// Segments that cross chunk ends: the chunk where such a segment begins (its
// last segment goes on, and did not itself begin earlier) adds the later
// chunks' carries in order and applies the update.
template <int DT, int EL, int C, int OPT>
__global__ __launch_bounds__(kBwdThreads) void seg_combine(MutTableArgs tabs, StateArgs state, float eps, int T, int D,
                                                           const int32_t* __restrict__ skeys,
                                                           const float* __restrict__ carry,
                                                           const float* __restrict__ head,
                                                           const float* __restrict__ wgcarry,
                                                           const int32_t* __restrict__ chunk_flags, long long nchunks,
                                                           float lr, SegOut so) {
  const int lane = threadIdx.x & (kWave - 1);
  const int lpr = D < kWave ? D : kWave;
  const int col = (lane % lpr) * EL;
  const long long k = static_cast<long long>(blockIdx.x) * (kBwdThreads / kWave) + (threadIdx.x >> 6);
  // the chunk's flags, last key and head sum are loaded before the segment
  // outputs are written, so that their round trip overlaps that step's (a wave
  // past the last chunk, or whose chunk is not full, reads in-bounds stand-ins
  // and uses none of them)
  const long long kc = k < nchunks ? k : nchunks - 1;
  const long long qlast = kc * C + C - 1 < so.n ? kc * C + C - 1 : so.n - 1;
  const int f = chunk_flags[kc];
  const int key = skeys[qlast];
  RowVec<EL> acc;
  acc.load(head + static_cast<size_t>(kc) * D + col);
  if (so.hcount) write_segments<C>(so, skeys, nchunks);  // uniform: every thread reaches its barrier
  if (k >= nchunks) return;
  if (!(f & kChunkLastCont)) return;
  // the chunk's last segment began inside it unless the chunk holds a single
  // segment that began earlier (then an earlier chunk owns it)
  if ((f & kChunkSingle) && (f & kChunkFirstCont)) return;
  // a chunk whose last segment goes on is full of valid keys, so key (the one
  // at the chunk's last position) is that segment's
  // Chunk j's first part is this segment's; the segment goes on past chunk j
  // only if chunk j holds nothing else and its last segment continues. The
  // last chunk it reaches is found 64 flags at a time (one per lane), then,
  // past those, 256 at a time (four per lane, loaded together), so a segment
  // spanning hundreds of chunks costs a few dependent loads, not one per chunk.
  long long last = nchunks - 1;
  bool found = false;
  {
    const long long jj = k + 1 + lane;
    const int fj = jj < nchunks ? chunk_flags[jj] : 0;
    const unsigned long long ends = __ballot(!((fj & kChunkSingle) && (fj & kChunkLastCont)));
    if (ends) {
      const long long e = k + __ffsll(static_cast<long long>(ends));
      last = e < last ? e : last;
      found = true;
    }
  }
  constexpr int kFlagLoads = 4;
  for (long long j = k + 1 + kWave; !found && j < nchunks; j += kFlagLoads * kWave) {
    int fj[kFlagLoads];
#pragma unroll
    for (int u = 0; u < kFlagLoads; ++u) {
      const long long jj = j + u * kWave + lane;
      fj[u] = jj < nchunks ? chunk_flags[jj] : 0;
    }
#pragma unroll
    for (int u = 0; u < kFlagLoads; ++u) {
      const unsigned long long ends = __ballot(!((fj[u] & kChunkSingle) && (fj[u] & kChunkLastCont)));
      if (!found && ends) {
        const long long e = j + u * kWave + __ffsll(static_cast<long long>(ends)) - 1;
        last = e < last ? e : last;
        found = true;
      }
    }
  }
  // The carries to add: chunks k+1..last. Every chunk strictly between k and
  // last lies wholly inside the segment, so each reduce workgroup whose four
  // chunks all do (w with k < 4w and 4w + 3 < last) left their sum in
  // wgcarry[w]; the others' carries are added one by one. Item i of the
  // sequence [chunks k+1 .. 4wa) [workgroups wa .. wb) [chunks 4wb .. last]
  // (or just chunks k+1 .. last) is at item_row(i).
  constexpr int kWaves = kBwdThreads / kWave;  // chunks per reduce workgroup
  const long long a0 = k + 1;
  long long wa = (a0 + kWaves - 1) / kWaves, wb = last / kWaves;
  if (wb <= wa) wa = wb = 0;
  const long long nh = wb > wa ? kWaves * wa - a0 : 0;
  const long long nw = wb - wa;
  const long long t0 = wb > wa ? kWaves * wb : a0;
  const long long nitems = nh + nw + (last - t0 + 1);
  auto item_row = [&](long long i) -> const float* {
    if (i < nh) return carry + static_cast<size_t>(a0 + i) * D;
    if (i < nh + nw) return wgcarry + static_cast<size_t>(wa + i - nh) * D;
    return carry + static_cast<size_t>(t0 + i - nh - nw) * D;
  };
  if constexpr (EL <= 4) {
    // D <= 256: the items summed R = 256 / D at a time, 4 columns per lane
    // (slot q of a load holds items q, q+R, ...), with 8 loads in flight; then the R slot sums are added in a fixed
    // butterfly order and each lane takes its own columns. A Zipf-hot row
    // whose carries span hundreds of chunks thus costs R times fewer round
    // trips than one carry per load (multi-hot backward 152.8 -> 148.0 us;
    // 16 loads in flight took 128 VGPRs and measured 153.6 us).
    const int lr = D >> 2;  // lanes per carry row
    const int R = kWave / lr;
    const int q = lane / lr;
    const int c4 = (lane - q * lr) * 4;
    constexpr int G = 8;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (long long j = 0; j < nitems; j += static_cast<long long>(R) * G) {
      float4 x[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const long long jj = j + static_cast<long long>(g) * R + q;
        x[g] = *reinterpret_cast<const float4*>(item_row(jj < nitems ? jj : nitems - 1) + c4);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if (j + static_cast<long long>(g) * R + q < nitems) {
          s.x += x[g].x;
          s.y += x[g].y;
          s.z += x[g].z;
          s.w += x[g].w;
        }
      }
    }
    for (int o = lr; o < kWave; o <<= 1) {
      s.x += __shfl_xor(s.x, o, kWave);
      s.y += __shfl_xor(s.y, o, kWave);
      s.z += __shfl_xor(s.z, o, kWave);
      s.w += __shfl_xor(s.w, o, kWave);
    }
#pragma unroll
    for (int e = 0; e < EL; ++e) {
      const int cc = col + e;  // column cc is component cc % 4 of lane cc / 4's sum
      const int src = cc >> 2;
      const float vx = __shfl(s.x, src, kWave), vy = __shfl(s.y, src, kWave);
      const float vz = __shfl(s.z, src, kWave), vw = __shfl(s.w, src, kWave);
      const int comp = cc & 3;
      acc.v[e] += comp == 0 ? vx : comp == 1 ? vy : comp == 2 ? vz : vw;
    }
  } else {
    // the items added in order; 4 loads in flight
    constexpr int G = 4;
    for (long long j = 0; j < nitems; j += G) {
      RowVec<EL> x[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const long long jj = j + g < nitems ? j + g : nitems - 1;
        x[g].load(item_row(jj) + col);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if (j + g < nitems) {
#pragma unroll
          for (int e = 0; e < EL; ++e) acc.v[e] += x[g].v[e];
        }
      }
    }
  }
  row_update<DT, EL, OPT>(tabs, state, eps, T, D, key, col, acc, lr);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct WsLayout {
  size_t d_pooled, keys_a, keys_b, vals_a, vals_b, bag_of, src_bag, counts, digit_off, row_total, partial, pos, uniq, seg,
      nuniq;
  size_t carry, head, wgcarry, chunk_flags, hcount, hwg, total;
};

// Gradient columns per lane for a row of D fp32 values, and the chunk of sorted
// occurrences one wave reduces (its gradient rows and table rows stay in
// registers: 2 * C * EL of them).
constexpr int seg_el(int D) { return D >= kWave ? D / kWave : 1; }
constexpr int seg_chunk(int el) { return el <= 1 ? 32 : 32 / el; }

// Digit width and pass count of the sort: 8-bit digits, or 9-bit ones where
// they need one pass fewer.
struct RadixPlan {
  int bits, passes;
};

RadixPlan radix_plan(int64_t total_rows) {
  int bits = 0;
  while ((1ll << bits) <= total_rows) ++bits;  // sentinel key = total_rows must fit
  const int p8 = (bits + 7) / 8, p9 = (bits + 8) / 9;
  return p9 < p8 ? RadixPlan{9, p9} : RadixPlan{8, p8};
}

WsLayout layout(int T, int B, int D, int64_t nnz) {
  WsLayout L{};
  const size_t n = static_cast<size_t>(nnz);
  const size_t ntiles = (n + kRadixTile - 1) / kRadixTile;
  const size_t ncounts = ntiles * kMaxRadixBins;
  const size_t scan_max = std::max(n, ncounts) + 1;
  size_t o = 0;
  L.d_pooled = o; o = align_up(o + static_cast<size_t>(B) * T * D * 4);
  L.keys_a = o; o = align_up(o + n * 4);
  L.keys_b = o; o = align_up(o + n * 4);
  L.vals_a = o; o = align_up(o + n * 4);
  L.vals_b = o; o = align_up(o + n * 4);
  L.bag_of = o; o = align_up(o + n * 4);
  L.src_bag = o; o = align_up(o + n * 4);
  L.counts = o; o = align_up(o + ncounts * 4);
  L.digit_off = o; o = align_up(o + (ncounts + 1) * 4);
  L.row_total = o; o = align_up(o + kMaxRadixBins * 4);
  L.partial = o; o = align_up(o + (scan_chunks(static_cast<long long>(scan_max)) + 1) * 8);
  L.pos = o; o = align_up(o + (n + 1) * 4);
  L.uniq = o; o = align_up(o + n * 4);
  L.seg = o; o = align_up(o + (n + 1) * 4);
  L.nuniq = o; o = align_up(o + 4);
  const size_t C = static_cast<size_t>(seg_chunk(seg_el(D)));
  const size_t nchunks = (n + C - 1) / C;
  L.carry = o; o = align_up(o + nchunks * D * 4);
  L.head = o; o = align_up(o + nchunks * D * 4);
  L.wgcarry = o; o = align_up(o + (nchunks + 3) / 4 * D * 4);
  L.chunk_flags = o; o = align_up(o + nchunks * 4);
  L.hcount = o; o = align_up(o + nchunks * 4);
  L.hwg = o; o = align_up(o + (nchunks + 3) / 4 * 4);
  L.total = o;
  return L;
}

template <int DT, int EL>
hipError_t launch_seg_reduce(const BwdArgs& a, const WsLayout& L, char* ws, const int32_t* skeys, int32_t sentinel,
                             const int32_t* src_bag, const float* d_pooled, const SegOut& so, hipStream_t st) {
  constexpr int C = seg_chunk(EL);
  const long long nchunks = (a.nnz + C - 1) / C;
  float* carry = reinterpret_cast<float*>(ws + L.carry);
  float* head = reinterpret_cast<float*>(ws + L.head);
  float* wgcarry = reinterpret_cast<float*>(ws + L.wgcarry);
  int32_t* flags = reinterpret_cast<int32_t*>(ws + L.chunk_flags);
  constexpr int kWavesPerBlock = kBwdThreads / kWave;
  const dim3 g(static_cast<unsigned>((nchunks + kWavesPerBlock - 1) / kWavesPerBlock)), blk(kBwdThreads);
  if (a.opt == kRowwiseAdagrad) {
    hipLaunchKernelGGL((seg_reduce_chunks<DT, EL, C, kRowwiseAdagrad>), g, blk, 0, st, a.tabs, a.state, a.eps, a.T, a.D,
                       skeys, a.nnz, sentinel, src_bag, d_pooled, a.T * a.B, a.lr, carry, head, wgcarry, flags, nchunks,
                       so.hcount, so.hwg);
    if (const hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    hipLaunchKernelGGL((seg_combine<DT, EL, C, kRowwiseAdagrad>), g, blk, 0, st, a.tabs, a.state, a.eps, a.T, a.D, skeys,
                       carry, head, wgcarry, flags, nchunks, a.lr, so);
  } else {
    hipLaunchKernelGGL((seg_reduce_chunks<DT, EL, C, kSgd>), g, blk, 0, st, a.tabs, a.state, a.eps, a.T, a.D, skeys,
                       a.nnz, sentinel, src_bag, d_pooled, a.T * a.B, a.lr, carry, head, wgcarry, flags, nchunks, so.hcount,
                       so.hwg);
    if (const hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    hipLaunchKernelGGL((seg_combine<DT, EL, C, kSgd>), g, blk, 0, st, a.tabs, a.state, a.eps, a.T, a.D, skeys, carry, head,
                       wgcarry, flags, nchunks, a.lr, so);
  }
  return hipGetLastError();
}

template <int DT>
hipError_t launch_reduce_dt(const BwdArgs& a, const WsLayout& L, char* ws, const int32_t* skeys, int32_t sentinel,
                            const int32_t* src_bag, const float* d_pooled, const SegOut& so, hipStream_t st) {
  switch (seg_el(a.D)) {
    case 1: return launch_seg_reduce<DT, 1>(a, L, ws, skeys, sentinel, src_bag, d_pooled, so, st);
    case 2: return launch_seg_reduce<DT, 2>(a, L, ws, skeys, sentinel, src_bag, d_pooled, so, st);
    case 4: return launch_seg_reduce<DT, 4>(a, L, ws, skeys, sentinel, src_bag, d_pooled, so, st);
    case 8: return launch_seg_reduce<DT, 8>(a, L, ws, skeys, sentinel, src_bag, d_pooled, so, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// LDS of one sample's interaction backward: Z [F][D+4] and S [Fp][F] fp32
static size_t ibwd_lds(int T, int D) {
  const int F = T + 1;
  return (static_cast<size_t>(F) * (D + 4) + static_cast<size_t>((F + 3) & ~3) * F) * 4;
}

constexpr size_t kLdsPerWorkgroup = 160 * 1024;
// room for the alignment of the dynamic LDS segment after a kernel's static one
constexpr size_t kLdsSlack = 256;

hipError_t launch_interact_bwd(int T, int B, int D, int layout, const float* e0, const float* pooled,
                               const float* d_out, float* d_e0, float* d_pooled, hipStream_t st) {
  const size_t lds = ibwd_lds(T, D);
  if (lds > kLdsPerWorkgroup) return hipErrorInvalidValue;
  const IbwdShare ia{T, D, (layout & DLRM_PAIRS_SELF) != 0, (layout & DLRM_WITH_EMBEDDINGS) != 0, e0, pooled,
                     d_out, d_pooled, d_e0, 0, B};
  hipLaunchKernelGGL(interact_bwd_kernel, dim3(B), dim3(kBwdThreads), lds, st, ia);
  return hipGetLastError();
}

size_t bwd_workspace_bytes(int T, int B, int D, int64_t nnz, int64_t /*total_rows*/) {
  return layout(T, B, D, nnz).total;
}

// How a backward call runs, decided on the host from the sizes alone.
// The per-table sort takes batches of at most one tile of occurrences per table
// on average (a longer table range still sorts, tile by tile through the
// workspace) and batches whose bags per table its bag loop walks quickly.
constexpr int kTableMaxBatch = 65536;


BwdPlanInfo bwd_plan(int T, int B, int D, int64_t nnz, int64_t total_rows, int64_t max_rows, bool want_segments) {
  BwdPlanInfo p{};
  const RadixPlan rp = radix_plan(total_rows);
  p.radix_bits = rp.bits;
  p.passes = nnz > 0 ? rp.passes : 0;
  const long long red_chunks = (nnz + seg_chunk(seg_el(D)) - 1) / seg_chunk(seg_el(D));
  p.fused_seg = nnz > 0 && want_segments && red_chunks <= kFusedSegChunks;
  p.seg_one_pass = nnz > 0 && want_segments && !p.fused_seg && scan_chunks(nnz) <= kScanThreads;
  const size_t ilds = ibwd_lds(T, D);
  p.table_sort = nnz > 0 && nnz <= static_cast<int64_t>(T) * kTableTile && B <= kTableMaxBatch;
  if (p.table_sort) {
    // row indices in [0, rows_t], an out-of-range index taking rows_t
    int bits = 0;
    while ((1ll << bits) <= max_rows) ++bits;
    p.radix_bits = 8;
    p.passes = (bits + 7) / 8;
    // the interaction backward's samples ride on table_sort, whose own
    // workgroups use the same dynamic LDS segment
    p.ibwd_shared = ilds <= kLdsPerWorkgroup;
    p.ibwd_lds = ilds;
    p.max_lds = std::max(sizeof(TableSortLds), ilds);
    return p;
  }
  // the interaction backward's samples ride on the scatter launches (and the
  // one-pass segment build) as extra workgroups when one sample's LDS fits
  // beside those kernels' own static LDS; otherwise it is a launch of its own
  size_t host_static = rp.bits == 9 ? sizeof(ScatterLds<9>) : sizeof(ScatterLds<8>);
  if (p.seg_one_pass && sizeof(SegChunkedLds) > host_static) host_static = sizeof(SegChunkedLds);
  p.ibwd_shared = nnz > 0 && host_static + kLdsSlack + ilds <= kLdsPerWorkgroup;
  p.ibwd_lds = ilds;
  p.max_lds = p.ibwd_shared ? host_static + kLdsSlack + ilds : (ilds > host_static ? ilds : host_static);
  return p;
}

hipError_t launch_embbag_bwd_update(const BwdArgs& a, hipStream_t st) {
  const WsLayout L = layout(a.T, a.B, a.D, a.nnz);
  char* ws = static_cast<char*>(a.workspace);
  float* d_pooled = reinterpret_cast<float*>(ws + L.d_pooled);
  int32_t* keys[2] = {reinterpret_cast<int32_t*>(ws + L.keys_a), reinterpret_cast<int32_t*>(ws + L.keys_b)};
  int32_t* vals[2] = {reinterpret_cast<int32_t*>(ws + L.vals_a), reinterpret_cast<int32_t*>(ws + L.vals_b)};
  int32_t* bag_of = reinterpret_cast<int32_t*>(ws + L.bag_of);
  int32_t* src_bag = reinterpret_cast<int32_t*>(ws + L.src_bag);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
  int32_t* digit_off = reinterpret_cast<int32_t*>(ws + L.digit_off);
  int32_t* row_total = reinterpret_cast<int32_t*>(ws + L.row_total);
  long long* partial = reinterpret_cast<long long*>(ws + L.partial);
  int32_t* pos = reinterpret_cast<int32_t*>(ws + L.pos);
  int32_t* uniq = a.unique_keys ? a.unique_keys : reinterpret_cast<int32_t*>(ws + L.uniq);
  int32_t* seg = a.seg_offsets ? a.seg_offsets : reinterpret_cast<int32_t*>(ws + L.seg);
  int32_t* nuniq = a.num_unique ? a.num_unique : reinterpret_cast<int32_t*>(ws + L.nuniq);

  const long long n = a.nnz;
  const bool want_segments = a.unique_keys || a.seg_offsets || a.num_unique;
  int max_rows = 0;
  for (int t = 0; t < a.T; ++t) max_rows = std::max(max_rows, static_cast<int>(a.tabs.rows[t]));
  const BwdPlanInfo plan = bwd_plan(a.T, a.B, a.D, n, a.total_rows, max_rows, want_segments);
  const size_t ilds = plan.ibwd_lds;
  if (ilds > kLdsPerWorkgroup) return hipErrorInvalidValue;
  hipError_t e = hipSuccess;
  // every launch is checked before the next is queued: a later step must not
  // run on the outputs of one that was never launched
#define DLRM_CHECK_LAUNCH()                      \
  do {                                           \
    if ((e = hipGetLastError()) != hipSuccess) { \
      return e;                                  \
    }                                            \
  } while (0)
  if (n == 0 || !plan.ibwd_shared) {  // 1. interaction backward as a launch of its own
    e = launch_interact_bwd(a.T, a.B, a.D, a.layout, a.e0, a.pooled, a.d_out, a.d_e0, d_pooled, st);
    if (e != hipSuccess) return e;
    if (n == 0) {  // no keys
      hipLaunchKernelGGL(zero_segments, dim3(1), dim3(64), 0, st, seg, nuniq);
      return hipGetLastError();
    }
  }
  // 1. otherwise the interaction backward's samples are shared out as extra
  // workgroups over the sort passes' scatter launches (the longest of the
  // sort; a share takes about as long as a scatter, and much longer than a
  // count) and the one-pass segment build when that runs, or over the two
  // launches of the per-table sort; nothing before the reduce reads its outputs
  const int passes = plan.passes;
  const bool fused_seg = plan.fused_seg;
  const long long nscan = scan_chunks(n);
  const bool seg_one_pass = plan.seg_one_pass;
  const int nshare = !plan.ibwd_shared || plan.table_sort ? 0 : passes + (seg_one_pass ? 1 : 0);
  int ishare = 0;
  const IbwdShare none{a.T, a.D, false, false, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 0};
  auto share = [&]() {
    if (nshare == 0) return none;
    IbwdShare ia{a.T, a.D, (a.layout & DLRM_PAIRS_SELF) != 0, (a.layout & DLRM_WITH_EMBEDDINGS) != 0, a.e0, a.pooled,
                 a.d_out, d_pooled, a.d_e0, 0, 0};
    ia.first = static_cast<int>(static_cast<long long>(a.B) * ishare / nshare);
    ia.count = static_cast<int>(static_cast<long long>(a.B) * (ishare + 1) / nshare) - ia.first;
    ++ishare;
    return ia;
  };
  // dynamic LDS only for a launch that carries interaction-backward workgroups
  auto share_lds = [&](const IbwdShare& ia) -> size_t { return ia.count > 0 ? ilds : 0; };
  const int32_t sentinel = static_cast<int32_t>(a.total_rows);
  const int32_t* skeys = nullptr;
  if (plan.table_sort) {  // 2-3. per table
    int32_t* tvalid = counts;
    int32_t* tbound = counts + a.T;
    int32_t* ws_uniq = reinterpret_cast<int32_t*>(ws + L.uniq);
    const TableSortArgs ts{a.T,    a.B,     a.offsets, a.indices, n,      keys[1], vals[1], pos,      tvalid,
                           tbound, keys[0], vals[0],   src_bag,   ws_uniq, bag_of, keys[0], src_bag, a.perm,
                           sentinel, a.status};
    // every interaction-backward sample rides on table_sort: its table
    // workgroups run about as long as the samples (splitting the samples with
    // table_place measured 1-2 us slower per step on the 26-table batch)
    const IbwdShare ia_sort =
        plan.ibwd_shared ? IbwdShare{a.T, a.D, (a.layout & DLRM_PAIRS_SELF) != 0, (a.layout & DLRM_WITH_EMBEDDINGS) != 0,
                                     a.e0, a.pooled, a.d_out, d_pooled, a.d_e0, 0, a.B}
                         : none;
    const size_t sort_lds = std::max(sizeof(TableSortLds), share_lds(ia_sort));
    hipLaunchKernelGGL(table_sort, dim3(a.T + ia_sort.count), dim3(kBwdThreads), sort_lds, st, ts, a.tabs, ia_sort);
    DLRM_CHECK_LAUNCH();
    hipLaunchKernelGGL(table_place, dim3(a.T), dim3(kBwdThreads), 0, st, keys[1], vals[1], pos, tvalid, tbound, a.tabs,
                       a.T, n, sentinel, keys[0], a.perm, src_bag);
    DLRM_CHECK_LAUNCH();
    skeys = keys[0];
  } else {
  // 2. keys
  {
    const long long nb = static_cast<long long>(a.T) * a.B;
    const long long avg = n / nb;  // lanes per bag: the average bag length, rounded down to a power of two
    const int lg = avg >= 64 ? 64 : avg >= 32 ? 32 : avg >= 16 ? 16 : avg >= 8 ? 8 : avg >= 4 ? 4 : avg >= 2 ? 2 : 1;
    const int own = static_cast<int>((nb * lg + kBwdThreads - 1) / kBwdThreads);
    const dim3 g(static_cast<unsigned>(own)), blk(kBwdThreads);
#define DLRM_BUILD_KEYS(L) \
  hipLaunchKernelGGL(build_keys<L>, g, blk, 0, st, a.tabs, a.T, a.B, a.offsets, a.indices, n, sentinel, keys[0], \
                     vals[0], bag_of, a.status, own, none)
    switch (lg) {
      case 64: DLRM_BUILD_KEYS(64); break;
      case 32: DLRM_BUILD_KEYS(32); break;
      case 16: DLRM_BUILD_KEYS(16); break;
      case 8: DLRM_BUILD_KEYS(8); break;
      case 4: DLRM_BUILD_KEYS(4); break;
      case 2: DLRM_BUILD_KEYS(2); break;
      default: DLRM_BUILD_KEYS(1); break;
    }
#undef DLRM_BUILD_KEYS
    DLRM_CHECK_LAUNCH();
  }
  // 3. radix sort, plan.radix_bits (8 or 9) bits per pass
  const int ntiles = static_cast<int>((n + kRadixTile - 1) / kRadixTile);
  int cur = 0;
  for (int p = 0; p < passes; ++p) {
    const int shift = p * plan.radix_bits;
    const bool inline_scan = ntiles <= kInlineScanTiles;
    // the last pass writes the permutation straight to the caller's array, if any
    int32_t* vout = (p + 1 == passes && a.perm) ? a.perm : vals[cur ^ 1];
    // ... and each sorted position's bag (for the reduce)
    const bool last_pass = p + 1 == passes;
    const IbwdShare ia_scatter = share();
    const dim3 gs(ntiles + ia_scatter.count), blk(kBwdThreads);
#define DLRM_SORT_PASS(BITS)                                                                                          \
  do {                                                                                                                \
    hipLaunchKernelGGL(radix_count<BITS>, dim3(ntiles), blk, 0, st, keys[cur], n, shift, ntiles, counts, none);       \
    DLRM_CHECK_LAUNCH();                                                                                              \
    if (!inline_scan) {                                                                                               \
      hipLaunchKernelGGL(radix_row_scan, dim3(1 << (BITS)), dim3(kScanThreads), 0, st, counts, ntiles, digit_off,      \
                         row_total);                                                                                  \
      DLRM_CHECK_LAUNCH();                                                                                            \
    }                                                                                                                 \
    hipLaunchKernelGGL(radix_scatter<BITS>, gs, blk, share_lds(ia_scatter), st, keys[cur], vals[cur], n, shift,       \
                       ntiles, counts, inline_scan ? nullptr : digit_off, row_total, keys[cur ^ 1], vout, bag_of,     \
                       last_pass ? src_bag : nullptr, ia_scatter);                                                    \
    DLRM_CHECK_LAUNCH();                                                                                              \
  } while (0)
    if (plan.radix_bits == 9) DLRM_SORT_PASS(9);
    else DLRM_SORT_PASS(8);
#undef DLRM_SORT_PASS
    cur ^= 1;
  }
  skeys = keys[cur];
  // plan.passes >= 1, so the last pass wrote a.perm (if given) and src_bag
  }
  // 4. segments: outputs only (the reduce reads the sorted keys), so built only
  // when the caller asks for any of them
  if (want_segments && !fused_seg) {
    const long long m = nscan;
    if (seg_one_pass) {  // chunk totals, then one pass that scans and builds the segments
      hipLaunchKernelGGL((scan_chunk_totals<HeadIn>), dim3(static_cast<unsigned>(m)), dim3(kScanThreads), 0, st,
                         HeadIn{skeys, sentinel}, n, partial);
      DLRM_CHECK_LAUNCH();
      const IbwdShare ia_seg = plan.table_sort ? none : share();
      hipLaunchKernelGGL(build_segments_chunked, dim3(static_cast<unsigned>(m) + ia_seg.count), dim3(kScanThreads),
                         share_lds(ia_seg), st, skeys, n, sentinel, partial, pos, uniq, seg, nuniq,
                         static_cast<int>(m), ia_seg);
      DLRM_CHECK_LAUNCH();
    } else {
      e = device_exclusive_scan(HeadIn{skeys, sentinel}, n, pos, partial, a.status, 0, st);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(build_segments, dim3(static_cast<unsigned>((n + kBwdThreads - 1) / kBwdThreads)),
                         dim3(kBwdThreads), 0, st, skeys, n, sentinel, pos, uniq, seg, nuniq);
      DLRM_CHECK_LAUNCH();
    }
  }
#undef DLRM_CHECK_LAUNCH
  // 5. reduce + SGD (and the segment outputs with fused_seg)
  const SegOut so = fused_seg ? SegOut{reinterpret_cast<int32_t*>(ws + L.hcount), reinterpret_cast<int32_t*>(ws + L.hwg),
                                       uniq, seg, nuniq, n, sentinel}
                              : SegOut{nullptr, nullptr, nullptr, nullptr, nullptr, n, sentinel};
  switch (a.dtype) {
    case DLRM_F32: return launch_reduce_dt<DLRM_F32>(a, L, ws, skeys, sentinel, src_bag, d_pooled, so, st);
    case DLRM_F16: return launch_reduce_dt<DLRM_F16>(a, L, ws, skeys, sentinel, src_bag, d_pooled, so, st);
    case DLRM_BF16: return launch_reduce_dt<DLRM_BF16>(a, L, ws, skeys, sentinel, src_bag, d_pooled, so, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dlrm
