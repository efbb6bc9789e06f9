// C ABI of libdlrm_embbag: argument validation on the host, then kernel
// launches on the caller's stream. Every check here runs before the first HIP
// call, so a rejected call touches neither the device nor any output.
#include <algorithm>
#include <stdint.h>
#include <string.h>

#include <vector>

#include "launch.h"

namespace {

using namespace dlrm;

constexpr int64_t kI32Max = 0x7fffffffLL;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int dtype_bytes(int dtype) {
  switch (dtype) {
    case DLRM_F32: return 4;
    case DLRM_F16:
    case DLRM_BF16: return 2;
    case DLRM_Q4:
    case DLRM_Q8T: return 1;
    default: return 0;
  }
}

int from_hip(hipError_t e) { return e == hipSuccess ? DLRM_OK : DLRM_E_HIP; }

// Checks shared by the forward and the backward.
int check_batch(int32_t T, int32_t B, int32_t D, int32_t dtype, const void* const* tables, const int64_t* rows,
                const int32_t* offsets, const int32_t* indices, int64_t nnz) {
  if (T < 1 || B < 1 || D < 1 || nnz < 0) return DLRM_E_INVAL;
  if (!tables || !rows || !offsets || (nnz > 0 && !indices)) return DLRM_E_INVAL;
  if (T > DLRM_MAX_TABLES) return DLRM_E_UNSUPPORTED;
  if (dtype_bytes(dtype) == 0) return DLRM_E_UNSUPPORTED;
  if (fwd_supported_row_bytes(D, dtype) == 0) return DLRM_E_UNSUPPORTED;
  if (static_cast<int64_t>(T) * B + 1 > kI32Max || nnz >= kI32Max) return DLRM_E_INVAL;
  for (int t = 0; t < T; ++t) {
    if (!tables[t] || rows[t] < 1 || rows[t] >= kI32Max) return DLRM_E_INVAL;
    if (!aligned(tables[t], 16)) return DLRM_E_ALIGN;
  }
  if (!aligned(offsets, 4) || (indices && !aligned(indices, 4))) return DLRM_E_ALIGN;
  return DLRM_OK;
}

// LDS bytes of the fused forward / standalone interaction tile for one sample.
size_t tile_bytes(int T, int D) {
  const size_t Fpad = static_cast<size_t>((T + 1 + 3) & ~3);
  return Fpad * (static_cast<size_t>(D) + 4) * 4 + static_cast<size_t>(T) * 2 * 4;
}

size_t bwd_lds_bytes(int T, int D) {
  const size_t F = static_cast<size_t>(T) + 1;
  return (F * (static_cast<size_t>(D) + 4) + ((F + 3) & ~static_cast<size_t>(3)) * F) * 4;  // S padded to 4-row blocks
}

constexpr size_t kLds = 160 * 1024;

// Floats per sample of the interaction output in a given layout.
int64_t out_width(int T, int D, int layout) {
  const int64_t F = T + 1;
  const int64_t P = (layout & DLRM_PAIRS_SELF) ? F * (F + 1) / 2 : F * (F - 1) / 2;
  return ((layout & DLRM_WITH_EMBEDDINGS) ? F * D : D) + P;
}

}  // namespace

namespace {

int bwd_update(int32_t T, int32_t B, int32_t D, int32_t dtype, void* const* tables, const int64_t* rows,
               const int32_t* offsets, const int32_t* indices, int64_t nnz, const float* e0, const float* pooled,
               const float* d_out, int layout, float lr, int opt, float eps, float* const* state, float* d_e0,
               int32_t* unique_keys, int32_t* seg_offsets, int32_t* num_unique, int32_t* perm, void* workspace,
               size_t ws_bytes, int32_t* status, void* stream) {
  if (dtype == DLRM_Q4 || dtype == DLRM_Q8T) return DLRM_E_UNSUPPORTED;  // defined for fp32 / fp16 / bf16
  int rc = check_batch(T, B, D, dtype, const_cast<const void* const*>(tables), rows, offsets, indices, nnz);
  if (rc != DLRM_OK) return rc;
  if (!e0 || !pooled || !d_out || !workspace) return DLRM_E_INVAL;
  if (layout < 0 || layout > (DLRM_PAIRS_SELF | DLRM_WITH_EMBEDDINGS)) return DLRM_E_INVAL;
  if (!aligned(e0, 16) || !aligned(pooled, 16) || !aligned(d_out, 4) || !aligned(workspace, 256)) return DLRM_E_ALIGN;
  if (d_e0 && !aligned(d_e0, 16)) return DLRM_E_ALIGN;
  if (D % 4 != 0 || D > 512) return DLRM_E_UNSUPPORTED;
  if (bwd_lds_bytes(T, D) > kLds) return DLRM_E_UNSUPPORTED;
  if (opt == kRowwiseAdagrad) {
    if (!state || !(eps > 0.f)) return DLRM_E_INVAL;
    for (int t = 0; t < T; ++t)
      if (!state[t]) return DLRM_E_INVAL;
      else if (!aligned(state[t], 4)) return DLRM_E_ALIGN;
  }
  int64_t total = 0;
  for (int t = 0; t < T; ++t) total += rows[t];
  if (total >= kI32Max) return DLRM_E_UNSUPPORTED;  // keys and the sentinel are int32
  if (ws_bytes < bwd_workspace_bytes(T, B, D, nnz, total)) return DLRM_E_WORKSPACE;
  BwdArgs a;
  memset(&a, 0, sizeof(a));
  a.T = T; a.B = B; a.D = D; a.dtype = dtype;
  int64_t base = 0;
  for (int t = 0; t < T; ++t) {
    a.tabs.ptr[t] = tables[t];
    a.tabs.rows[t] = static_cast<int32_t>(rows[t]);
    a.tabs.base[t] = static_cast<int32_t>(base);
    base += rows[t];
    if (opt == kRowwiseAdagrad) a.state.ptr[t] = state[t];
  }
  a.total_rows = total;
  a.offsets = offsets; a.indices = indices; a.nnz = nnz;
  a.e0 = e0; a.pooled = pooled; a.d_out = d_out; a.lr = lr; a.opt = opt; a.eps = eps; a.d_e0 = d_e0;
  a.layout = layout;
  a.unique_keys = unique_keys; a.seg_offsets = seg_offsets; a.num_unique = num_unique; a.perm = perm;
  a.workspace = workspace; a.ws_bytes = ws_bytes; a.status = status;
  return from_hip(launch_embbag_bwd_update(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

const char* dlrm_status_string(int status) {
  switch (status) {
    case DLRM_OK: return "ok";
    case DLRM_E_INVAL: return "invalid argument";
    case DLRM_E_UNSUPPORTED: return "unsupported dtype, embedding dimension or table count";
    case DLRM_E_WORKSPACE: return "workspace too small";
    case DLRM_E_HIP: return "HIP runtime error";
    case DLRM_E_ALIGN: return "device pointer not 16-byte aligned";
    case DLRM_E_SCRATCH: return "batch needs more scratch than the allocation-free entry point holds";
    default: return "unknown status";
  }
}

int dlrm_version(void) { return 100; }  // 0.1.0

int dlrm_lengths_to_offsets(int64_t n, const int32_t* lengths, int32_t* offsets, int32_t* status, void* stream) {
  if (n < 0 || n >= kI32Max || !offsets || (n > 0 && !lengths)) return DLRM_E_INVAL;
  if (!aligned(offsets, 4) || (lengths && !aligned(lengths, 4))) return DLRM_E_ALIGN;
  return from_hip(launch_lengths_to_offsets(n, lengths, offsets, status, static_cast<hipStream_t>(stream)));
}

int dlrm_embbag_fwd(int32_t T, int32_t B, int32_t D, int32_t dtype, const void* const* tables, const int64_t* rows,
                    const int32_t* offsets, const int32_t* indices, int64_t nnz, const float* e0, float* out_pooled,
                    float* out_inter, int32_t* status, void* stream) {
  return dlrm_embbag_fwd_ex(T, B, D, dtype, tables, rows, offsets, indices, nnz, e0, out_pooled, out_inter, 0, status,
                            stream);
}

int dlrm_embbag_fwd_ex(int32_t T, int32_t B, int32_t D, int32_t dtype, const void* const* tables,
                       const int64_t* rows, const int32_t* offsets, const int32_t* indices, int64_t nnz,
                       const float* e0, float* out_pooled, float* out_inter, int32_t layout, int32_t* status,
                       void* stream) {
  if (dtype == DLRM_Q4 || dtype == DLRM_Q8T) return DLRM_E_UNSUPPORTED;  // quantized rows: dlrm_embbag_fwd_q4 / _q8t
  if (layout < 0 || layout > (DLRM_PAIRS_SELF | DLRM_WITH_EMBEDDINGS)) return DLRM_E_INVAL;
  int rc = check_batch(T, B, D, dtype, tables, rows, offsets, indices, nnz);
  if (rc != DLRM_OK) return rc;
  if (static_cast<int64_t>(B) * out_width(T, D, layout) >= (int64_t(1) << 40)) return DLRM_E_INVAL;
  if (!out_pooled && !out_inter) return DLRM_E_INVAL;
  if (out_inter && !e0) return DLRM_E_INVAL;
  if (out_pooled && !aligned(out_pooled, 16)) return DLRM_E_ALIGN;
  if (out_inter && (!aligned(out_inter, 4) || !aligned(e0, 16))) return DLRM_E_ALIGN;
  if (out_inter && fwd_lds_bytes(T, D, dtype) > kLds) return DLRM_E_UNSUPPORTED;
  FwdArgs a;
  memset(&a, 0, sizeof(a));
  a.T = T; a.B = B; a.D = D; a.dtype = dtype;
  for (int t = 0; t < T; ++t) {
    a.tabs.ptr[t] = tables[t];
    a.tabs.rows[t] = static_cast<int32_t>(rows[t]);
  }
  a.offsets = offsets; a.indices = indices; a.nnz = nnz;
  a.e0 = e0; a.out_pooled = out_pooled; a.out_inter = out_inter; a.status = status; a.layout = layout;
  return from_hip(launch_embbag_fwd(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Shared by the two quantized forwards: same checks, same launch; scale_bias is
// the table-wise (scale, bias) array, or null for row-wise codes.
int fwd_quantized(int32_t dtype, int32_t T, int32_t B, int32_t D, const void* const* tables, const float* scale_bias,
             const int64_t* rows, const int32_t* offsets, const int32_t* indices, int64_t nnz, const float* e0,
             float* out_pooled, float* out_inter, int32_t* status, void* stream) {
  int rc = check_batch(T, B, D, dtype, tables, rows, offsets, indices, nnz);
  if (rc != DLRM_OK) return rc;
  if (D != 128 && D != 256 && D != 512) return DLRM_E_UNSUPPORTED;
  if (!out_inter || !e0) return DLRM_E_INVAL;
  if (dtype == DLRM_Q8T && !scale_bias) return DLRM_E_INVAL;
  if (out_pooled && !aligned(out_pooled, 16)) return DLRM_E_ALIGN;
  if (!aligned(out_inter, 4) || !aligned(e0, 16)) return DLRM_E_ALIGN;
  if (fwd_lds_bytes(T, D, dtype) > kLds) return DLRM_E_UNSUPPORTED;
  FwdArgs a;
  memset(&a, 0, sizeof(a));
  a.T = T; a.B = B; a.D = D; a.dtype = dtype;
  for (int t = 0; t < T; ++t) {
    a.tabs.ptr[t] = tables[t];
    a.tabs.rows[t] = static_cast<int32_t>(rows[t]);
    if (dtype == DLRM_Q8T) {
      a.qscale[t] = scale_bias[2 * t];
      a.qbias[t] = scale_bias[2 * t + 1];
    }
  }
  a.offsets = offsets; a.indices = indices; a.nnz = nnz;
  a.e0 = e0; a.out_pooled = out_pooled; a.out_inter = out_inter; a.status = status;
  return from_hip(launch_embbag_fwd(a, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int dlrm_embbag_fwd_q4(int32_t T, int32_t B, int32_t D, const void* const* tables, const int64_t* rows,
                       const int32_t* offsets, const int32_t* indices, int64_t nnz, const float* e0,
                       float* out_pooled, float* out_inter, int32_t* status, void* stream) {
  return fwd_quantized(DLRM_Q4, T, B, D, tables, nullptr, rows, offsets, indices, nnz, e0, out_pooled, out_inter,
                       status, stream);
}

int dlrm_embbag_fwd_q8t(int32_t T, int32_t B, int32_t D, const void* const* tables, const float* scale_bias,
                        const int64_t* rows, const int32_t* offsets, const int32_t* indices, int64_t nnz,
                        const float* e0, float* out_pooled, float* out_inter, int32_t* status, void* stream) {
  return fwd_quantized(DLRM_Q8T, T, B, D, tables, scale_bias, rows, offsets, indices, nnz, e0, out_pooled, out_inter,
                  status, stream);
}

int dlrm_interact_ex(int32_t T, int32_t B, int32_t D, int32_t layout, const float* e0, const float* pooled,
                     float* out, void* stream) {
  if (T < 1 || B < 1 || D < 1 || !e0 || !pooled || !out) return DLRM_E_INVAL;
  if (layout < 0 || layout > (DLRM_PAIRS_SELF | DLRM_WITH_EMBEDDINGS)) return DLRM_E_INVAL;
  if (T > DLRM_MAX_TABLES || D % 4 != 0 || D > 1024) return DLRM_E_UNSUPPORTED;
  if (static_cast<int64_t>(B) * out_width(T, D, layout) >= (int64_t(1) << 40)) return DLRM_E_INVAL;
  if (!aligned(e0, 16) || !aligned(pooled, 16) || !aligned(out, 4)) return DLRM_E_ALIGN;
  if (tile_bytes(T, D) > kLds) return DLRM_E_UNSUPPORTED;
  return from_hip(launch_interact(T, B, D, layout, e0, pooled, out, static_cast<hipStream_t>(stream)));
}

int dlrm_interact(int32_t T, int32_t B, int32_t D, const float* e0, const float* pooled, float* out, void* stream) {
  return dlrm_interact_ex(T, B, D, 0, e0, pooled, out, stream);
}

int dlrm_interact_bwd(int32_t T, int32_t B, int32_t D, int32_t layout, const float* e0, const float* pooled,
                      const float* d_out, float* d_e0, float* d_pooled, void* stream) {
  if (T < 1 || B < 1 || D < 1 || !e0 || !pooled || !d_out || !d_pooled) return DLRM_E_INVAL;
  if (layout < 0 || layout > (DLRM_PAIRS_SELF | DLRM_WITH_EMBEDDINGS)) return DLRM_E_INVAL;
  if (T > DLRM_MAX_TABLES || D % 4 != 0 || D > 512) return DLRM_E_UNSUPPORTED;
  if (static_cast<int64_t>(B) * out_width(T, D, layout) >= (int64_t(1) << 40)) return DLRM_E_INVAL;
  if (!aligned(e0, 16) || !aligned(pooled, 16) || !aligned(d_out, 4) || !aligned(d_pooled, 16)) return DLRM_E_ALIGN;
  if (d_e0 && !aligned(d_e0, 16)) return DLRM_E_ALIGN;
  if (bwd_lds_bytes(T, D) > kLds) return DLRM_E_UNSUPPORTED;
  return from_hip(launch_interact_bwd(T, B, D, layout, e0, pooled, d_out, d_e0, d_pooled,
                                      static_cast<hipStream_t>(stream)));
}

int dlrm_embbag_bwd_workspace_bytes(int32_t T, int32_t B, int32_t D, int64_t nnz, const int64_t* rows, size_t* bytes) {
  if (T < 1 || B < 1 || D < 1 || nnz < 0 || nnz >= kI32Max || !bytes) return DLRM_E_INVAL;
  if (T > DLRM_MAX_TABLES) return DLRM_E_UNSUPPORTED;
  int64_t total = 0;
  if (rows)
    for (int t = 0; t < T; ++t) total += rows[t];
  *bytes = bwd_workspace_bytes(T, B, D, nnz, total);
  return DLRM_OK;
}


int dlrm_embbag_bwd_update(int32_t T, int32_t B, int32_t D, int32_t dtype, void* const* tables, const int64_t* rows,
                           const int32_t* offsets, const int32_t* indices, int64_t nnz, const float* e0,
                           const float* pooled, const float* d_out, float lr, float* d_e0, int32_t* unique_keys,
                           int32_t* seg_offsets, int32_t* num_unique, int32_t* perm, void* workspace, size_t ws_bytes,
                           int32_t* status, void* stream) {
  return bwd_update(T, B, D, dtype, tables, rows, offsets, indices, nnz, e0, pooled, d_out, 0, lr, kSgd, 0.f, nullptr,
                    d_e0, unique_keys, seg_offsets, num_unique, perm, workspace, ws_bytes, status, stream);
}

int dlrm_embbag_bwd_update_noalloc(int32_t T, int32_t B, int32_t D, int32_t dtype, void* const* tables,
                                   const int64_t* rows, const int32_t* offsets, const int32_t* indices, int64_t nnz,
                                   const float* e0, const float* pooled, const float* d_out, float lr, float* d_e0,
                                   int32_t* unique_keys, int32_t* seg_offsets, int32_t* num_unique, int32_t* perm,
                                   int32_t* status, void* stream) {
  // size first (host only): a batch beyond the array is rejected before any HIP call
  if (T < 1 || B < 1 || D < 1 || nnz < 0 || nnz >= kI32Max || !rows) return DLRM_E_INVAL;
  if (T > DLRM_MAX_TABLES) return DLRM_E_UNSUPPORTED;
  int64_t total = 0;
  for (int t = 0; t < T; ++t) total += rows[t];
  const size_t need = bwd_workspace_bytes(T, B, D, nnz, total);
  if (need > kNoAllocScratchBytes) return DLRM_E_SCRATCH;
  void* ws = nullptr;
  if (noalloc_scratch(&ws) != hipSuccess) return DLRM_E_HIP;
  return bwd_update(T, B, D, dtype, tables, rows, offsets, indices, nnz, e0, pooled, d_out, 0, lr, kSgd, 0.f, nullptr,
                    d_e0, unique_keys, seg_offsets, num_unique, perm, ws, kNoAllocScratchBytes, status, stream);
}

int dlrm_embbag_bwd_update_adagrad(int32_t T, int32_t B, int32_t D, int32_t dtype, void* const* tables,
                                   const int64_t* rows, const int32_t* offsets, const int32_t* indices, int64_t nnz,
                                   const float* e0, const float* pooled, const float* d_out, float lr, float eps,
                                   float* const* row_state, float* d_e0, int32_t* unique_keys, int32_t* seg_offsets,
                                   int32_t* num_unique, int32_t* perm, void* workspace, size_t ws_bytes,
                                   int32_t* status, void* stream) {
  return bwd_update(T, B, D, dtype, tables, rows, offsets, indices, nnz, e0, pooled, d_out, 0, lr, kRowwiseAdagrad, eps,
                    row_state, d_e0, unique_keys, seg_offsets, num_unique, perm, workspace, ws_bytes, status, stream);
}

int dlrm_embbag_bwd_plan(int32_t T, int32_t B, int32_t D, int64_t nnz, const int64_t* rows, int32_t want_segments,
                         int32_t* plan) {
  if (T < 1 || B < 1 || D < 1 || nnz < 0 || nnz >= kI32Max || !rows || !plan) return DLRM_E_INVAL;
  if (T > DLRM_MAX_TABLES) return DLRM_E_UNSUPPORTED;
  int64_t total = 0, max_rows = 0;
  for (int t = 0; t < T; ++t) {
    if (rows[t] < 1 || rows[t] >= kI32Max) return DLRM_E_INVAL;
    total += rows[t];
    max_rows = std::max(max_rows, rows[t]);
  }
  if (total >= kI32Max) return DLRM_E_UNSUPPORTED;
  const BwdPlanInfo p = bwd_plan(T, B, D, nnz, total, max_rows, want_segments != 0);
  plan[0] = p.radix_bits;
  plan[1] = p.passes;
  plan[2] = p.ibwd_shared ? 1 : 0;
  plan[3] = static_cast<int32_t>(p.max_lds);
  plan[4] = p.table_sort ? 1 : 0;
  return p.ibwd_lds > kLds ? DLRM_E_UNSUPPORTED : DLRM_OK;
}

int dlrm_embbag_bwd_update_ex(int32_t T, int32_t B, int32_t D, int32_t dtype, void* const* tables,
                              const int64_t* rows, const int32_t* offsets, const int32_t* indices, int64_t nnz,
                              const float* e0, const float* pooled, const float* d_out, int32_t layout, float lr,
                              float eps, float* const* row_state, float* d_e0, int32_t* unique_keys,
                              int32_t* seg_offsets, int32_t* num_unique, int32_t* perm, void* workspace,
                              size_t ws_bytes, int32_t* status, void* stream) {
  return bwd_update(T, B, D, dtype, tables, rows, offsets, indices, nnz, e0, pooled, d_out, layout, lr,
                    row_state ? kRowwiseAdagrad : kSgd, eps, row_state, d_e0, unique_keys, seg_offsets, num_unique,
                    perm, workspace, ws_bytes, status, stream);
}

int dlrm_validate_bags(int32_t T, int32_t B, const int64_t* rows, const int32_t* offsets, const int32_t* indices,
                       int64_t nnz) {
  if (T < 1 || B < 1 || nnz < 0 || !rows || !offsets || (nnz > 0 && !indices)) return DLRM_E_INVAL;
  const int64_t nb = static_cast<int64_t>(T) * B;
  int bits = 0;
  if (offsets[0] != 0 || offsets[nb] != nnz) bits |= DLRM_STATUS_BAD_OFFSETS;
  for (int64_t i = 0; i < nb; ++i) {
    const int64_t s0 = offsets[i], s1 = offsets[i + 1];
    if (s0 < 0 || s0 > nnz || s1 > nnz || s1 < s0) bits |= DLRM_STATUS_BAD_OFFSETS;
  }
  if (bits) return bits;
  for (int64_t i = 0; i < nb; ++i) {
    const int t = static_cast<int>(i / B);
    for (int64_t p = offsets[i]; p < offsets[i + 1]; ++p)
      if (indices[p] < 0 || indices[p] >= rows[t]) bits |= DLRM_STATUS_BAD_INDEX;
  }
  return bits;
}

}  // extern "C"
