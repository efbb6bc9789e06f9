/*
 * dlrm_probe.h -- measurement kernel of libdlrm_embbag.so, not part of the
 * method: the bare random-row gather that the fused forward's bandwidth is
 * compared against ("Terabyte Embedding Tables and Compute-Bound Neural Layers
 * Force Meta's DLRM to Split Training", section "The memory wall of sparse
 * features": the embedding lookups need almost no arithmetic but enormous
 * memory traffic, so the gather itself is the ceiling of the path).
 */
#ifndef DLRM_PROBE_H
#define DLRM_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads, for every position p of a table-major CSR batch, the whole row
 * indices[p] of its table (the same rows dlrm_embbag_fwd reads for that batch,
 * with the same one-row-per-wave-wide-load access), sums what each lane loaded
 * and writes one float per thread to sink, so that no load can be dropped.
 * Nothing else is read or written: no offsets per bag, no output rows.
 *   T, D, dtype, tables, rows, indices, nnz   as in dlrm_embbag_fwd (16-bit or fp32
 *            rows of 128 .. 1024 bytes); an index outside its table reads row 0
 *   table_start  host int64 [T + 1]: CSR position of each table's first occurrence
 *            (offsets[t * B] of the batch), table_start[T] = nnz
 *   sink     device fp32 [4096 * 256] (contents meaningless)
 * Returns a dlrm_status.
 */
int dlrm_probe_row_gather(int32_t T, int32_t D, int32_t dtype, const void* const* tables, const int64_t* rows,
                          const int64_t* table_start, const int32_t* indices, int64_t nnz, float* sink,
                          void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DLRM_PROBE_H */
