// Host-side interface between the C ABI (api.cpp) and the kernel launchers.
// Plain C++: no device code, so api.cpp builds as host code.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "dlrm_embbag.h"

namespace dlrm {

// Table pointers and row counts travel in the kernel arguments (1.5 KB for 128 tables),
// so a wave picks its table with a scalar load from the argument segment.
struct TableArgs {
  const void* ptr[DLRM_MAX_TABLES];
  int32_t rows[DLRM_MAX_TABLES];
};

struct MutTableArgs {
  void* ptr[DLRM_MAX_TABLES];
  int32_t rows[DLRM_MAX_TABLES];
  int32_t base[DLRM_MAX_TABLES];  // first global key of each table
};

// Per-row optimizer state (row-wise AdaGrad: one fp32 sum of squares per row).
struct StateArgs {
  float* ptr[DLRM_MAX_TABLES];
};

enum Optimizer { kSgd = 0, kRowwiseAdagrad = 1 };

struct FwdArgs {
  int T, B, D, dtype;
  TableArgs tabs;
  float qscale[DLRM_MAX_TABLES], qbias[DLRM_MAX_TABLES];  // DLRM_Q8T: per-table scale and bias
  const int32_t* offsets;
  const int32_t* indices;
  int64_t nnz;
  const float* e0;
  float* out_pooled;
  float* out_inter;
  int32_t* status;
  int layout;  // DLRM_PAIRS_SELF | DLRM_WITH_EMBEDDINGS bits of the interaction output
};

hipError_t launch_embbag_fwd(const FwdArgs& a, hipStream_t s);
hipError_t launch_interact(int T, int B, int D, int layout, const float* e0, const float* pooled, float* out,
                           hipStream_t s);
hipError_t launch_interact_bwd(int T, int B, int D, int layout, const float* e0, const float* pooled,
                               const float* d_out, float* d_e0, float* d_pooled, hipStream_t s);
hipError_t launch_lengths_to_offsets(int64_t n, const int32_t* lengths, int32_t* offsets, int32_t* status,
                                     hipStream_t s);

struct BwdArgs {
  int T, B, D, dtype;
  MutTableArgs tabs;
  int64_t total_rows;
  const int32_t* offsets;
  const int32_t* indices;
  int64_t nnz;
  const float* e0;
  const float* pooled;
  const float* d_out;
  float lr;
  int opt;     // Optimizer
  int layout;  // interaction output layout bits of d_out (DLRM_PAIRS_SELF, DLRM_WITH_EMBEDDINGS)
  float eps;   // row-wise AdaGrad: added to sqrt(state)
  StateArgs state;
  float* d_e0;
  int32_t* unique_keys;
  int32_t* seg_offsets;
  int32_t* num_unique;
  int32_t* perm;
  void* workspace;
  size_t ws_bytes;
  int32_t* status;
};

size_t bwd_workspace_bytes(int T, int B, int D, int64_t nnz, int64_t total_rows);

// Library-owned scratch of the allocation-free backward (one array per GPU).
constexpr size_t kNoAllocScratchBytes = size_t(DLRM_NOALLOC_SCRATCH_BYTES);
// Device address of the current device's array (looked up once per device).
hipError_t noalloc_scratch(void** ptr);

// How the sparse backward runs for given sizes (host only).
struct BwdPlanInfo {
  int radix_bits;    // digit width of the sort (8 or 9)
  int passes;        // sort passes (per-table sort: those of the table with the most rows)
  bool table_sort;   // occurrences sorted per table (two launches) instead of by radix passes
  bool fused_seg;    // segment outputs written by the reduce's combine step
  bool seg_one_pass; // segment outputs from chunk totals + one scan-and-write launch
  bool ibwd_shared;  // interaction backward rides on the sort launches (else its own launch)
  size_t ibwd_lds;   // LDS of one interaction-backward sample
  size_t max_lds;    // largest LDS of any workgroup of the call
};
BwdPlanInfo bwd_plan(int T, int B, int D, int64_t nnz, int64_t total_rows, int64_t max_rows, bool want_segments);
hipError_t launch_embbag_bwd_update(const BwdArgs& a, hipStream_t s);

// shared by forward and backward: fused/standalone interaction tile sizes
int fwd_supported_row_bytes(int D, int dtype);
// LDS bytes the fused forward needs for one workgroup (must be <= 160 KiB)
size_t fwd_lds_bytes(int T, int D, int dtype);

}  // namespace dlrm
