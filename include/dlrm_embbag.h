/*
 * dlrm_embbag.h -- C ABI of libdlrm_embbag.so, the MI355X (gfx950) hot path of
 * the DLRM recommendation model: multi-table embedding-bag pooling, the
 * pairwise dot-product feature interaction, and the sparse embedding backward
 * with an SGD update.
 *
 * Problem statement followed (web pages on DLRM):
 *   - "DLRM" note (vault-aram.pages.dev/Notes/DLRM), section 2 "The
 *     Architecture": one embedding table per categorical feature; each
 *     categorical ID selects one row; dense features pass through a bottom MLP
 *     whose output e_0 has the embedding dimension.
 *   - same note, section 3 "The Pairwise Interaction Layer": dot products
 *     e_i . e_j between the embeddings and e_0, concatenated with e_0. This
 *     library computes the variant without self-pairs that the section
 *     mentions: pairs i > j over Z = [e_0, e_1 .. e_T].
 *   - same note, section 9 "Weaknesses": history (multi-valued) features are
 *     aggregated before use; here a bag of IDs is sum-pooled.
 *   - same note, section 5 "Training": the embedding tables are trained; the
 *     update implemented here is plain SGD on the rows a batch touched.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *   T       number of tables (1 <= T <= DLRM_MAX_TABLES)
 *   B       batch size (samples), B >= 1
 *   D       embedding dimension; the row of a table is D elements of the table
 *           dtype, and D * sizeof(dtype) must be a power of two in [16, 1024]
 *           bytes (fp32: D in {4,8,...,256}; fp16/bf16: D in {8,...,512})
 *   F = T + 1 vectors per sample (e_0 then the T pooled embeddings)
 *   P = F (F - 1) / 2 interaction values per sample
 *   Bags are a single table-major CSR: bag (t, b) is
 *       indices[offsets[t*B + b] .. offsets[t*B + b + 1])
 *   i.e. the per-table CSRs laid end to end; offsets has T*B + 1 int32
 *   entries, offsets[0] = 0 and offsets[T*B] = nnz; indices are int32 row
 *   numbers in [0, rows[t]).
 *   Interaction output, per sample b (row-major [B][D + P], fp32):
 *       out[b][0 .. D)      = e0[b]  (bit copy)
 *       out[b][D + k]       = Z[b][i] . Z[b][j],  k = i (i - 1) / 2 + j,
 *                             0 <= j < i < F  (strict lower triangle, row-major)
 *   Pooled layout: pooled[b][t][d], fp32, [B][T][D].
 *
 * Pointers: "device" pointers are HIP device memory (hipMalloc / torch CUDA
 * tensors) aligned to 16 bytes; "host" pointers are ordinary CPU memory read
 * during the call only. The caller owns every buffer; the library keeps no
 * state between calls and allocates no device memory (the backward uses a
 * caller-provided workspace).
 *
 * Ordering: every call only enqueues work on `stream` (a hipStream_t; NULL is
 * the default stream) and returns without synchronising. Inputs must stay
 * unchanged, and outputs unread, until the stream has reached the work.
 *
 * Errors: argument errors are detected on the host before anything is
 * enqueued; the call then returns a negative dlrm_status and touches no
 * output. Data errors (an index outside its table, offsets that are not a
 * valid CSR) are detected on the device: the kernels never read out of bounds,
 * an out-of-range index contributes nothing, an invalid offset range counts as
 * an empty bag, and the matching DLRM_STATUS_* bit is OR-ed into *status
 * (device int32, may be NULL). The caller clears *status before the call.
 */
#ifndef DLRM_EMBBAG_H
#define DLRM_EMBBAG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DLRM_MAX_TABLES 128

typedef enum {
  DLRM_OK = 0,
  DLRM_E_INVAL = -1,       /* NULL where required, non-positive size, inconsistent sizes */
  DLRM_E_UNSUPPORTED = -2, /* dtype, D or T outside what the kernels handle */
  DLRM_E_WORKSPACE = -3,   /* workspace smaller than dlrm_embbag_bwd_workspace_bytes() */
  DLRM_E_HIP = -4,         /* a HIP runtime call or kernel launch failed */
  DLRM_E_ALIGN = -5,       /* a device pointer is not 16-byte aligned */
  DLRM_E_SCRATCH = -6      /* the batch needs more scratch than the allocation-free entry point holds */
} dlrm_status;

/* Bytes of the library-owned scratch array behind dlrm_embbag_bwd_update_noalloc (one per GPU). */
#define DLRM_NOALLOC_SCRATCH_BYTES (64u << 20)

/* DLRM_Q8T: table-wise 8-bit tables (only through dlrm_embbag_fwd_q8t): a row is D uint8 codes,
 * one (scale, bias) pair per table.
 * DLRM_Q4: row-wise 4-bit tables (only through dlrm_embbag_fwd_q4): a row is D 4-bit codes,
 * its fp32 scale and fp32 bias, padded to a power of two (see dlrm_embbag_fwd_q4).
 * (3 was a row-wise 8-bit format whose D + 8 byte rows straddle two 128-byte lines; it is
 * not offered: it was slower than the bf16 rows it compresses.) */
typedef enum { DLRM_F32 = 0, DLRM_F16 = 1, DLRM_BF16 = 2, DLRM_Q8T = 4, DLRM_Q4 = 5 } dlrm_dtype;

/* Interaction output layouts ("DLRM" note, section 3, The Pairwise Interaction
 * Layer): bits of the `layout` argument of dlrm_embbag_fwd_ex, dlrm_interact_ex
 * and dlrm_interact_bwd. 0 is the layout given at the top of this file.
 *   DLRM_PAIRS_SELF       the section's formula with the pairs of a vector with
 *                         itself: pairs i >= j, P = F (F + 1) / 2, pair (i, j) at
 *                         dot index i (i + 1) / 2 + j (row-major lower triangle
 *                         with the diagonal). Without it: i > j, i (i - 1) / 2 + j.
 *   DLRM_WITH_EMBEDDINGS  the variant the section mentions that concatenates the
 *                         original embeddings alongside the interaction vector:
 *                         out[b] = [Z[b][0] | Z[b][1] | .. | Z[b][T] | dots], i.e.
 *                         e0 then the T pooled vectors (F * D floats), then the P
 *                         dots. Without it: out[b] = [e0 | dots].
 * A sample's output row has W = (with embeddings ? F * D : D) + P floats. */
#define DLRM_PAIRS_SELF 1
#define DLRM_WITH_EMBEDDINGS 2

/* bits OR-ed into the device status word */
#define DLRM_STATUS_BAD_INDEX 1   /* an index outside [0, rows[t]) */
#define DLRM_STATUS_BAD_OFFSETS 2 /* offsets[0] != 0, a decrease, an offset outside [0, nnz], offsets[T*B] != nnz,
                                     or a negative bag length */

/* Human-readable name of a dlrm_status value. Never NULL. */
const char* dlrm_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int dlrm_version(void);

/*
 * Bag lengths -> CSR offsets (exclusive prefix sum).
 *   lengths  device int32 [n]      length of each bag (table-major order)
 *   offsets  device int32 [n + 1]  out: offsets[0] = 0, offsets[i+1] = offsets[i] + lengths[i]
 *   n        number of bags (T*B), 0 <= n < 2^31
 *   status   device int32 or NULL: DLRM_STATUS_BAD_OFFSETS if a length is negative (it then counts
 *            as 0) or the total exceeds INT32_MAX (offsets are then unspecified)
 * Uses no workspace: per-chunk totals are parked in `offsets` itself between its three kernels.
 */
int dlrm_lengths_to_offsets(int64_t n, const int32_t* lengths, int32_t* offsets, int32_t* status, void* stream);

/*
 * Embedding-bag forward, optionally fused with the interaction.
 * Defined by the "DLRM" note: section 2, The Architecture (one table per
 * categorical feature, an ID selects one row, the bottom MLP yields e_0 in the
 * embedding dimension); section 9, Weaknesses (a multi-valued feature is
 * aggregated: here the bag's rows are summed, an empty bag gives zeros); and
 * section 3, The Pairwise Interaction Layer (dot products of every pair of
 * Z = [e_0, pooled_1 .. pooled_T], concatenated with e_0; the variant without
 * self-pairs, i > j).
 *   T, B, D, dtype      as above
 *   tables   host array [T] of device pointers; table t is row-major [rows[t]][D] of dtype
 *   rows     host int64 [T], 1 <= rows[t] < 2^31
 *   offsets  device int32 [T*B + 1], indices device int32 [nnz], nnz (host) = offsets[T*B]
 *   e0       device fp32 [B][D]; required when out_inter != NULL, ignored otherwise
 *   out_pooled  device fp32 [B][T][D] or NULL: the pooled sums (fp32 accumulation)
 *   out_inter   device fp32 [B][D + P] or NULL: [e0 | strict-lower dots]; pooled vectors are
 *               kept on chip between the gather and the dots (nothing else is written)
 *   At least one of out_pooled / out_inter must be non-NULL.
 */
int dlrm_embbag_fwd(int32_t T, int32_t B, int32_t D, int32_t dtype, const void* const* tables,
                    const int64_t* rows, const int32_t* offsets, const int32_t* indices, int64_t nnz,
                    const float* e0, float* out_pooled, float* out_inter, int32_t* status, void* stream);

/*
 * dlrm_embbag_fwd with a choice of interaction layout (DLRM_PAIRS_SELF,
 * DLRM_WITH_EMBEDDINGS or both; "DLRM" note, section 3, The Pairwise
 * Interaction Layer: its formula includes the pairs of a vector with itself,
 * and some variants concatenate the original embeddings alongside the
 * interaction vector). The pooled vectors still stay on chip between the
 * gather and the dots; with DLRM_WITH_EMBEDDINGS they are written to out_inter
 * as part of the output row.
 *   out_inter   device fp32 [B][W], W as given with the layout bits
 *   layout      0 .. 3; every other argument as in dlrm_embbag_fwd (layout 0 is dlrm_embbag_fwd)
 */
int dlrm_embbag_fwd_ex(int32_t T, int32_t B, int32_t D, int32_t dtype, const void* const* tables,
                       const int64_t* rows, const int32_t* offsets, const int32_t* indices, int64_t nnz,
                       const float* e0, float* out_pooled, float* out_inter, int32_t layout, int32_t* status,
                       void* stream);

/*
 * The fused forward on row-wise 4-bit tables. The "Terabyte Embedding Tables..."
 * article (section "Scaling limits and the reality of production") reports
 * 4-bit integer quantization of the embedding vectors exchanged between
 * devices; here the same 4-bit codes, with a scale and a bias per row, are what
 * the tables store in HBM, so a lookup reads a quarter of the bf16 row's bytes
 * plus 8.
 * Row r of table t starts at byte r * S, S = the smallest power of two >= D/2 + 8
 * (128 for D = 128, 256 for D = 256, 512 for D = 512), so a row never straddles
 * more 128-byte lines than its size needs (one line for D = 128):
 *   bytes [0, D/2)        codes: byte k holds column 2k in its low 4 bits and
 *                         column 2k + 1 in its high 4 bits (q in 0..15)
 *   bytes [D/2, D/2 + 4)  fp32 scale s_r;  bytes [D/2 + 4, D/2 + 8)  fp32 bias c_r
 *   the rest              padding, never read
 *   value[d] = s_r * q[d] + c_r
 *   tables     host array [T] of device pointers (16-byte aligned), table t is uint8 [rows[t]][S]
 *   D          128, 256 or 512
 *   out_inter  required; out_pooled optional; everything else as in dlrm_embbag_fwd.
 * Pooling sums s_r * q per column in fp32 and adds the bag's summed biases.
 */
int dlrm_embbag_fwd_q4(int32_t T, int32_t B, int32_t D, const void* const* tables, const int64_t* rows,
                       const int32_t* offsets, const int32_t* indices, int64_t nnz, const float* e0,
                       float* out_pooled, float* out_inter, int32_t* status, void* stream);

/*
 * The fused forward on table-wise 8-bit tables: row r of table t is D uint8
 * codes, value[d] = scale_t * q[d] + bias_t with one (scale, bias) pair per
 * table, so a lookup reads exactly D bytes (one aligned 128-byte line for
 * D = 128) and nothing else. Coarser than row-wise codes (the step is the
 * table's range / 255), but no second read per lookup.
 *   tables      host array [T] of device pointers (16-byte aligned), table t is uint8 [rows[t]][D]
 *   scale_bias  host fp32 [T][2]: (scale_t, bias_t)
 *   D           128, 256 or 512; out_inter required; everything else as in dlrm_embbag_fwd.
 */
int dlrm_embbag_fwd_q8t(int32_t T, int32_t B, int32_t D, const void* const* tables, const float* scale_bias,
                        const int64_t* rows, const int32_t* offsets, const int32_t* indices, int64_t nnz,
                        const float* e0, float* out_pooled, float* out_inter, int32_t* status, void* stream);

/*
 * Interaction alone, from pooled vectors in HBM ("DLRM" note, section 3, The
 * Pairwise Interaction Layer: the dot products e_i . e_j of every pair i > j of
 * Z = [e_0, e_1 .. e_T], concatenated with e_0).
 *   e0 device fp32 [B][D], pooled device fp32 [B][T][D], out device fp32 [B][D + P]
 *   in the layout given at the top of this file. D must be a multiple of 4, at most 1024.
 */
int dlrm_interact(int32_t T, int32_t B, int32_t D, const float* e0, const float* pooled, float* out,
                  void* stream);

/*
 * Interaction alone with a choice of layout ("DLRM" note, section 3, The
 * Pairwise Interaction Layer: its formula takes the dot products e_i . e_j for
 * i <= j, self-pairs included; the section mentions variants without them and
 * variants that concatenate the original embeddings alongside the dots).
 *   layout  bits DLRM_PAIRS_SELF, DLRM_WITH_EMBEDDINGS (0 .. 3; 0 is dlrm_interact)
 *   e0 device fp32 [B][D], pooled device fp32 [B][T][D], out device fp32 [B][W]
 *   (W as given with the layout bits); the e0 and pooled values in the output are
 *   bit copies. D must be a multiple of 4, at most 1024.
 */
int dlrm_interact_ex(int32_t T, int32_t B, int32_t D, int32_t layout, const float* e0, const float* pooled,
                     float* out, void* stream);

/*
 * Backward of dlrm_interact_ex, for a caller that owns the layers above (a top
 * MLP) and the optimizer of the pooled vectors. The gradient of Z_i . Z_j is
 * Z_j for Z_i and Z_i for Z_j, so with g the upstream gradient of the pairs,
 * S the symmetric F x F matrix holding g at (i, j) and (j, i) (2 g on the
 * diagonal for self-pairs, 0 there otherwise): dZ[b] = S[b] Z[b] + the direct
 * gradient of the Z rows that appear in the output themselves (e0 always; with
 * DLRM_WITH_EMBEDDINGS every row).
 *   layout    the forward's layout bits (0 .. 3)
 *   e0 device fp32 [B][D], pooled device fp32 [B][T][D]   (the forward's inputs)
 *   d_out     device fp32 [B][W]: dL/d(out) in the layout of dlrm_interact_ex
 *   d_e0      device fp32 [B][D] or NULL: out, dZ[:, 0]
 *   d_pooled  device fp32 [B][T][D]: out, dZ[:, 1 .. T]
 * D must be a multiple of 4, at most 512; (T + 1)(D + 4 + T + 1) * 4 bytes of LDS
 * must fit in 160 KB.
 */
int dlrm_interact_bwd(int32_t T, int32_t B, int32_t D, int32_t layout, const float* e0, const float* pooled,
                      const float* d_out, float* d_e0, float* d_pooled, void* stream);

/*
 * Workspace needed by dlrm_embbag_bwd_update for these sizes (bytes, written to *bytes).
 */
int dlrm_embbag_bwd_workspace_bytes(int32_t T, int32_t B, int32_t D, int64_t nnz, const int64_t* rows,
                                    size_t* bytes);

/*
 * Sparse backward of the forward above followed by an SGD step on the touched rows.
 * The "DLRM" note, section 5, Training, has the embedding tables trained with
 * the rest of the model; the pages give no backward, so this is the exact
 * gradient of dlrm_embbag_fwd's [e0 | dots]: dZ[b] = S[b] Z[b] with S[b] the
 * symmetric matrix of the upstream pair gradients, then for each table row the
 * sum of dZ over the bags that hold it (a bag holding the row k times counts it
 * k times), then W <- W - lr * G (plain SGD, no momentum or decay).
 *   tables   host array [T] of device pointers, updated in place: for every row r of table t
 *            that the batch references, W_t[r] <- W_t[r] - lr * G, G = sum over the occurrences
 *            of (t, r) of dL/dpooled[b][t] (fp32 sum in a fixed order, result rounded to dtype).
 *            Rows not referenced are not written.
 *   rows, offsets, indices, nnz   as in the forward (same batch)
 *   e0       device fp32 [B][D], pooled device fp32 [B][T][D] (the forward's out_pooled)
 *   d_out    device fp32 [B][D + P]: dL/d(out_inter)
 *   lr       learning rate
 *   d_e0     device fp32 [B][D] or NULL: out, dL/de0 = d_out[:, :D] + sum_j g_{0j} Z_j
 *   unique_keys  device int32 [nnz] or NULL: out, sorted distinct global rows
 *                (key = rows[0] + ... + rows[t-1] + r) in the first U entries
 *   seg_offsets  device int32 [nnz + 1] or NULL: out, occurrences of unique_keys[u] are
 *                perm[seg_offsets[u] .. seg_offsets[u+1]); seg_offsets[U] is the number of
                occurrences with a valid index (= nnz for a valid batch; occurrences with an
                out-of-range index are sorted after every valid one and belong to no segment)
 *   num_unique   device int32 [1] or NULL: out, U
 *                (the three segment outputs are built only when at least one is requested)
 *   perm     device int32 [nnz] or NULL: out, the stable order of occurrences by key
 *            (ties keep CSR order); this permutation is unique. Occurrences with an
 *            out-of-range index come last, in CSR order
 *   workspace, ws_bytes  device scratch of at least dlrm_embbag_bwd_workspace_bytes() bytes
 *            (no initial contents needed)
 * Requires sum(rows) < 2^31. Deterministic: identical inputs give bit-identical outputs.
 * Occurrences with an out-of-range index are dropped (and DLRM_STATUS_BAD_INDEX set).
 * With offsets that are not a valid CSR (DLRM_STATUS_BAD_OFFSETS set) every access still
 * stays in bounds and rows that no index names are not written, but where bags overlap
 * (decreasing offsets) the outputs and the update are unspecified.
 */
int dlrm_embbag_bwd_update(int32_t T, int32_t B, int32_t D, int32_t dtype, void* const* tables,
                           const int64_t* rows, const int32_t* offsets, const int32_t* indices, int64_t nnz,
                           const float* e0, const float* pooled, const float* d_out, float lr, float* d_e0,
                           int32_t* unique_keys, int32_t* seg_offsets, int32_t* num_unique, int32_t* perm,
                           void* workspace, size_t ws_bytes, int32_t* status, void* stream);

/*
 * The sparse backward for a forward run with an interaction layout (the
 * general form of dlrm_embbag_bwd_update and dlrm_embbag_bwd_update_adagrad).
 * d_out is the gradient of dlrm_embbag_fwd_ex's output in that layout ("DLRM"
 * note, section 3: self-pairs, and the embeddings concatenated alongside the
 * dots, whose own gradient then adds to the pooled vectors' and to e0's).
 *   layout     0 .. 3 (DLRM_PAIRS_SELF | DLRM_WITH_EMBEDDINGS); d_out is device fp32 [B][W]
 *   row_state  NULL: SGD (eps unused); else row-wise AdaGrad as in dlrm_embbag_bwd_update_adagrad
 * Every other argument, the outputs and the determinism as in dlrm_embbag_bwd_update.
 */
int dlrm_embbag_bwd_update_ex(int32_t T, int32_t B, int32_t D, int32_t dtype, void* const* tables,
                              const int64_t* rows, const int32_t* offsets, const int32_t* indices, int64_t nnz,
                              const float* e0, const float* pooled, const float* d_out, int32_t layout, float lr,
                              float eps, float* const* row_state, float* d_e0, int32_t* unique_keys,
                              int32_t* seg_offsets, int32_t* num_unique, int32_t* perm, void* workspace,
                              size_t ws_bytes, int32_t* status, void* stream);

/*
 * dlrm_embbag_bwd_update for callers that cannot allocate device memory (code
 * under graph capture, tight serving loops, harnesses that forbid it): the
 * same arguments minus the workspace, the same results bit for bit. The scratch
 * the call needs lives in a static device array of DLRM_NOALLOC_SCRATCH_BYTES
 * (64 MiB) that the library owns; each GPU the library runs on holds its own
 * copy until the process ends. The call allocates nothing (no hipMalloc, no
 * library routine that allocates).
 *   Returns DLRM_E_SCRATCH, touching nothing, when dlrm_embbag_bwd_workspace_bytes()
 *   for these sizes exceeds DLRM_NOALLOC_SCRATCH_BYTES (for D = 128 fp32 gradients
 *   that is about 2,000 samples of 26 tables).
 * Every call on one GPU shares that GPU's array, which keeps the last call's contents
 * (the call needs none of them): calls that overlap on one GPU (different streams,
 * or threads) race and must be serialised by the caller.
 */
int dlrm_embbag_bwd_update_noalloc(int32_t T, int32_t B, int32_t D, int32_t dtype, void* const* tables,
                                   const int64_t* rows, const int32_t* offsets, const int32_t* indices, int64_t nnz,
                                   const float* e0, const float* pooled, const float* d_out, float lr, float* d_e0,
                                   int32_t* unique_keys, int32_t* seg_offsets, int32_t* num_unique, int32_t* perm,
                                   int32_t* status, void* stream);

/*
 * The same backward with a row-wise AdaGrad step instead of SGD ("DLRM" note,
 * section 5, Training: the optimizer is typically adaptive, Adam or AdaGrad,
 * and its state is sharded with the tables). The state is one fp32 value per
 * table row, the running sum of the row's mean squared gradient:
 *     s_r <- s_r + (1/D) sum_d G[r][d]^2,    W_r <- W_r - lr * G_r / (sqrt(s_r) + eps)
 * for every row r the batch references (G as in dlrm_embbag_bwd_update; rows not
 * referenced keep both W and s).
 *   row_state  host array [T] of device fp32 pointers, table t's state is [rows[t]],
 *              read and updated in place (start from zeros, or any non-negative values)
 *   eps        > 0
 * Every other argument as in dlrm_embbag_bwd_update. Deterministic.
 */
int dlrm_embbag_bwd_update_adagrad(int32_t T, int32_t B, int32_t D, int32_t dtype, void* const* tables,
                                   const int64_t* rows, const int32_t* offsets, const int32_t* indices, int64_t nnz,
                                   const float* e0, const float* pooled, const float* d_out, float lr, float eps,
                                   float* const* row_state, float* d_e0, int32_t* unique_keys, int32_t* seg_offsets,
                                   int32_t* num_unique, int32_t* perm, void* workspace, size_t ws_bytes,
                                   int32_t* status, void* stream);

/*
 * How dlrm_embbag_bwd_update / _adagrad will run for these sizes. Host only:
 * no GPU call, nothing enqueued. plan is host int32 [5]:
 *   plan[0]  digit width of the radix sort of the occurrences (8 or 9 bits)
 *   plan[1]  sort passes (0 when nnz = 0; with plan[4] set, the passes of the
 *            table with the most rows)
 *   plan[2]  1 when the interaction backward's samples run as extra workgroups
 *            of the sort's launches, 0 when it is a launch of its own (one
 *            sample's LDS does not fit beside the sort kernel's within 160 KiB)
 *   plan[3]  largest LDS of any workgroup of the call, in bytes
 *   plan[4]  1 when the occurrences are sorted per table (nnz <= 2048 * T and
 *            B <= 65536: one workgroup sorts each table's occurrences by row,
 *            a second launch places them), 0 for the radix sort over all keys
 *   want_segments  nonzero when the call will ask for unique_keys, seg_offsets or num_unique
 * Returns DLRM_E_UNSUPPORTED when one sample's interaction backward alone exceeds 160 KiB.
 */
int dlrm_embbag_bwd_plan(int32_t T, int32_t B, int32_t D, int64_t nnz, const int64_t* rows, int32_t want_segments,
                         int32_t* plan);

/*
 * Host-side check of a bag description (host arrays): returns the DLRM_STATUS_* bits the
 * device would report (0 = valid), or a negative dlrm_status for bad arguments.
 */
int dlrm_validate_bags(int32_t T, int32_t B, const int64_t* rows, const int32_t* offsets,
                       const int32_t* indices, int64_t nnz);

#ifdef __cplusplus
}
#endif
#endif /* DLRM_EMBBAG_H */
