/*
 * mhc_floor.h -- data-movement floors of the boundary's launch geometry, in libmhc_amd.so.
 *
 * These two calls compute nothing of the method. They exist so that the boundary's time
 * can be compared, through the same binding, stream and graph path, with what a kernel of
 * the same shape costs when it only moves the same bytes (mhc_floor_boundary_traffic) or
 * moves none (mhc_floor_empty). Conventions as in mhc.h: device pointers owned by the
 * caller, work enqueued on `stream`, every argument checked before any launch, status
 * codes from enum mhc_status.
 *
 * Geometry (the boundary's at up to 32 rows with two elements per lane, as mhc_boundary
 * launches a call that writes a layer input): workgroups of 512 threads, each owning
 * 1024 consecutive hidden elements (one chunk) of one row, ceil(H / 1024) chunks per row,
 * 8 * ceil(R / 8) * chunks workgroups in one launch, a row's chunks on workgroup ids
 * congruent to the row mod 8 (one XCD). Each lane owns one 4-byte vector (two bf16
 * elements) of the row.
 */
#ifndef MHC_AMD_FLOOR_H
#define MHC_AMD_FLOOR_H

#include <stdint.h>

#include "mhc.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * mhc_floor_boundary_traffic -- the bytes of mhc_boundary with an MXFP8 layer input, moved
 * with the boundary's geometry and access kind (non-temporal 4-byte loads and stores),
 * without its arithmetic or its row handoff. Each lane loads its vector of the T partial
 * slices and of the n = 4 streams, then stores four stream vectors, one layer-input
 * vector, two E4M3 bytes and, on every 16th lane, one scale byte. The stored words are
 * bitwise combinations (xor) of the loaded ones, so no load can be dropped; their values
 * mean nothing.
 *   x_partials [T, R, H], residual [R, 4, H] (bf16 bits, read);
 *   residual_out [R, 4, H], layer_input_out [R, H] (bf16 bits), mx_data_out [R, H],
 *   mx_scale_out [R, H / 32] (bytes) (written; none may overlap another argument).
 *   rows in [0, 65536] (0: no-op), tp in [1, 64], hidden in [32, 65536] and a multiple
 *   of 32, else MHC_ERR_SHAPE; a NULL pointer, MHC_ERR_INVALID_ARG; bf16 tensors not
 *   16-byte aligned or mx_data_out not 8-byte aligned, MHC_ERR_ALIGN; launch failure,
 *   MHC_ERR_HIP.
 */
int mhc_floor_boundary_traffic(const uint16_t* x_partials, int tp, const uint16_t* residual,
                               int rows, int hidden, uint16_t* residual_out,
                               uint16_t* layer_input_out, uint8_t* mx_data_out,
                               uint8_t* mx_scale_out, mhc_stream_t stream);

/*
 * mhc_floor_empty -- a kernel of the same grid and workgroup size as
 * mhc_floor_boundary_traffic for (rows, hidden) that does nothing: the cost of the launch
 * itself. rows in [0, 65536] (0: no-op), hidden as above, else MHC_ERR_SHAPE.
 */
int mhc_floor_empty(int rows, int hidden, mhc_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MHC_AMD_FLOOR_H */
