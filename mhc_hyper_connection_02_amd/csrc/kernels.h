// Internal interface between the C ABI (api.hip) and the kernel launchers.
// Arguments are validated by the caller; the launchers only enqueue work.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "coeff_epilogue.h"

namespace mhc {

// Row r's epoch (the call tag of its row handoff) sits at epoch[r * kEpochStride]: one
// 128-byte line per row, since rows that share a line run on different XCDs (measured:
// 0.25 us per 32-row boundary call with the epochs packed).
constexpr int kEpochStride = 32;

struct BoundaryLaunch {
  // exactly one sublayer-output source: x_partials (tp slices) or gemm2_permuted (finalize)
  const uint16_t* x_partials;
  int tp;
  const uint16_t* gemm2_permuted;
  int num_permuted;
  const float* expert_weights;
  const int32_t* idx;
  const uint16_t* shared_output;
  int top_k;
  const uint16_t* residual;
  uint16_t* residual_out;
  const float* post;
  const float* comb;
  const float* pre;             // NULL: residual-only
  const uint16_t* norm_weight;
  float eps;
  int rows, hidden;
  uint16_t* layer_input_out;
  uint8_t* mx_data_out;         // NULL: no MXFP8
  uint8_t* mx_scale_out;
  int scale_kt;                 // 0: scales row-major [rows][hidden/32]; else the swizzled
                                // 128x4 layout with scale_kt tiles per 128 rows
  unsigned long long* slots;    // [max_rows][slot_stride] row-RMS handoff words
  unsigned* epoch;              // [max_rows][kEpochStride]: row r's epoch at r * kEpochStride
  unsigned* errors;             // [1] handoff timeouts
  int slot_stride;
  int spin_limit;
  bool xcd_handoff;             // workgroups with ids congruent mod 8 share an XCD (probed at
                                // handle creation): row handoff words go through its L2
  int max_wgs_per_xcd;          // resident workgroups of this block size on one XCD
  int block;                    // 128, 256 or 512 threads per workgroup (layer-input kernels)
  int lane_elems;               // 4 or 2: the kernels that write a layer input run that many
                                // elements per lane at block_n = block * 8 / lane_elems threads
                                // (the same chunks per row); 8: block, eight per lane
  int block_n;
  int max_wgs_per_xcd_n;        // resident workgroups of block_n threads on one XCD
  int mode;                     // kBoundaryMix, kBoundaryFirst or kBoundaryHead
  // deferred coefficients (mix mode): post, comb and pre are computed in the kernel from a
  // pending coefficient call's split-K partials, and written to post/comb/pre by the
  // row's first workgroup
  bool defer;
  CoeffEpilogue coef;
  float* pre_pending;           // the pending call's pre output (written even residual-only)
};

// What the layer-input kernel computes (the layer input is always RMSNorm(y) * w):
//  mix:   x from the sublayer output, new streams s' = post x + comb s (stored),
//         y = sum_j pre_j s'_j
//  first: x = the one slice x_partials[0] (the embedding), every stream := x (stored),
//         y = x (the identity pre-mix); no streams read, no post/comb/pre
//  head:  no x; y = bf16(sum_j pre_j s_j) on the given streams; nothing stored but the
//         layer input (and its MXFP8 form)
constexpr int kBoundaryMix = 0;
constexpr int kBoundaryFirst = 1;
constexpr int kBoundaryHead = 2;

struct PreLaunch {
  const uint16_t* residual;
  const uint16_t* fn;
  const float* scale;
  const float* base;
  float rms_eps, pre_eps, sinkhorn_eps, post_alpha;
  int sinkhorn_iters, rows, hidden;
  float* pre_out;
  float* post_out;
  float* comb_out;
  float* part;                  // pre_scratch_floats(max_rows, hidden) floats
  int ks_count;                 // splits of `part`: 0 for the split-K plan's, else a multiple
                                // of 4 (partials written by the fused boundary)
};

// The boundary fused with the next coefficient call (boundary_tile.hip): the boundary's
// launch (mix mode, with a layer input) plus the coefficient call's arguments.
struct TileLaunch {
  BoundaryLaunch b;
  const uint16_t* fn;           // [4 * hidden][24] bf16
  CoeffEpilogue coef;           // scale, base, K, eps, alpha, iters (part unused)
  float* next_pre;
  float* next_post;
  float* next_comb;
  float* part_out;              // non-NULL: write the next coefficients' partials here
                                // (coeff_part_index, ks = boundary_tile_part_ks(hidden)) and finish none
  bool defer_in;                // b.post, b.comb and b.pre are a pending call's outputs: finish
                                // them from in_coef.part (another fused kernel's part_out;
                                // requires part_out) and write them, instead of reading them
  CoeffEpilogue in_coef;
  unsigned long long* words;    // boundary_tile_words(tile_rows, hidden) tagged partials
  int tile_rows;                // rows the words cover (the handle's), >= the call's rows
  int wgs_per_xcd;              // resident workgroups of the tile kernel on one XCD
  bool spread;                  // chunk c of every tile on XCD c % 8 (else a tile per XCD)
};
int boundary_tile_resident_wgs_per_cu();
int boundary_tile_chunks(int hidden);
size_t boundary_tile_words(int rows, int hidden);
int boundary_tile_part_ks(int hidden);
bool boundary_tile_fits(int hidden, int wgs_per_xcd);
hipError_t launch_boundary_tile(const TileLaunch& T, hipStream_t stream);

// chunks of a row: ceil(hidden / 8 / block), `block` 16-byte vectors per workgroup
int boundary_chunks(int hidden, int block);
// Row-handoff words per row: one per wave at the most waves a row can have (the
// 128-thread chunks at 512 threads), rounded up to 16 (a 128-byte line).
int boundary_handoff_words(int hidden);
int boundary_resident_wgs_per_cu(int block);
hipError_t launch_boundary(const BoundaryLaunch& L, hipStream_t stream);
hipError_t launch_collapse_mean(const uint16_t* streams, int rows, int hidden, uint16_t* out,
                                hipStream_t stream);

void pre_plan(int rows, int hidden, int* ks_count, int* steps_per_wg, int* rows_pad);
size_t pre_scratch_floats_for(int rows, int hidden);
hipError_t launch_pre_coeffs(const PreLaunch& L, hipStream_t stream);   // both kernels
hipError_t launch_pre_partial(const PreLaunch& L, hipStream_t stream);   // split-K only
hipError_t launch_pre_epilogue(const PreLaunch& L, hipStream_t stream);  // epilogue only
CoeffEpilogue pre_epilogue_args(const PreLaunch& L);

hipError_t launch_fill_u32(unsigned* p, size_t n, unsigned value, hipStream_t stream);

// Whether the device deals workgroup ids round-robin to its 8 XCDs (ids congruent mod 8 on one
// XCD), read from the hardware's XCC id register over a grid of the size the kernels use;
// `buf` holds kXcdProbeWgs words of device memory.
constexpr int kXcdProbeWgs = 512;
hipError_t probe_xcd_round_robin(unsigned* buf, bool* round_robin);

}  // namespace mhc
