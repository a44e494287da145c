// Data-movement floors of the boundary's launch geometry (include/mhc_floor.h): the same
// grid, workgroup size, workgroup-to-(row, chunk) placement and access kind as the
// boundary at up to 32 rows, with its bytes moved and nothing computed, and the same grid
// doing nothing at all. They compute nothing of the method; they tell how much of a
// boundary call's time any kernel of its shape pays.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "mhc_floor.h"

namespace {

using mhc::load_nt;
using mhc::store_nt;

constexpr int kFloorBlock = 512;                // threads per workgroup
constexpr int kFloorChunk = 2 * kFloorBlock;    // hidden elements per workgroup
constexpr int kFloorXcds = 8;
constexpr int kFloorMaxTp = 64;
constexpr int kFloorMaxRows = 65536;
constexpr int kFloorMaxHidden = 65536;

struct FloorParams {
  const uint32_t* xp;        // [tp][rows][nv]
  const uint32_t* res_in;    // [rows][4][nv]
  uint32_t* res_out;         // [rows][4][nv]
  uint32_t* layer_out;       // [rows][nv]
  uint16_t* mx_data;         // [rows][nv] (two E4M3 bytes per vector)
  uint8_t* mx_scale;         // [rows][hidden / 32]
  int tp, rows, nv, chunks;  // nv: 4-byte vectors per row
};

inline int floor_chunks(int hidden) { return (hidden + kFloorChunk - 1) / kFloorChunk; }
inline int floor_grid(int rows, int hidden) {
  return kFloorXcds * ((rows + kFloorXcds - 1) / kFloorXcds) * floor_chunks(hidden);
}

__global__ __launch_bounds__(kFloorBlock) void floor_boundary_kernel(const FloorParams p) {
  const int wg = blockIdx.x;
  const int local = wg / kFloorXcds;
  const int c = local % p.chunks;
  const int r = (local / p.chunks) * kFloorXcds + wg % kFloorXcds;
  if (r >= p.rows) return;  // uniform per workgroup
  const int v = c * kFloorBlock + threadIdx.x;
  const bool active = v < p.nv;
  const int va = active ? v : 0;  // every load in bounds, results of idle lanes dropped
  uint32_t s[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) s[j] = load_nt(p.res_in + ((size_t)r * 4 + j) * p.nv + va);
  uint32_t x = 0;
  const uint32_t* src = p.xp + (size_t)r * p.nv + va;
  const size_t slice = (size_t)p.rows * p.nv;
  for (int t0 = 0; t0 < p.tp; t0 += 8) {
    uint32_t xv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (t0 + u < p.tp) xv[u] = load_nt(src + (size_t)(t0 + u) * slice);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (t0 + u < p.tp) x ^= xv[u];
  }
  if (!active) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) store_nt(p.res_out + ((size_t)r * 4 + i) * p.nv + v, s[i] ^ x);
  const uint32_t y = s[0] ^ s[1] ^ s[2] ^ s[3] ^ x;
  store_nt(p.layer_out + (size_t)r * p.nv + v, y);
  store_nt(p.mx_data + (size_t)r * p.nv + v, (uint16_t)(y ^ (y >> 16)));
  if ((v & 15) == 0) p.mx_scale[(size_t)r * (p.nv / 16) + v / 16] = (uint8_t)y;
}

__global__ __launch_bounds__(kFloorBlock) void floor_empty_kernel(const FloorParams) {}

inline bool aligned(const void* q, unsigned a) {
  return (reinterpret_cast<uintptr_t>(q) % a) == 0;
}

inline bool shape_ok(int rows, int hidden) {
  return rows >= 0 && rows <= kFloorMaxRows && hidden >= 32 && hidden <= kFloorMaxHidden &&
         hidden % 32 == 0;
}

}  // namespace

extern "C" int mhc_floor_boundary_traffic(const uint16_t* x_partials, int tp,
                                          const uint16_t* residual, int rows, int hidden,
                                          uint16_t* residual_out, uint16_t* layer_input_out,
                                          uint8_t* mx_data_out, uint8_t* mx_scale_out,
                                          mhc_stream_t stream) {
  if (!shape_ok(rows, hidden) || tp < 1 || tp > kFloorMaxTp) return MHC_ERR_SHAPE;
  if (rows == 0) return MHC_OK;
  if (!x_partials || !residual || !residual_out || !layer_input_out || !mx_data_out ||
      !mx_scale_out)
    return MHC_ERR_INVALID_ARG;
  if (!aligned(x_partials, 16) || !aligned(residual, 16) || !aligned(residual_out, 16) ||
      !aligned(layer_input_out, 16) || !aligned(mx_data_out, 8))
    return MHC_ERR_ALIGN;
  FloorParams p;
  p.xp = reinterpret_cast<const uint32_t*>(x_partials);
  p.res_in = reinterpret_cast<const uint32_t*>(residual);
  p.res_out = reinterpret_cast<uint32_t*>(residual_out);
  p.layer_out = reinterpret_cast<uint32_t*>(layer_input_out);
  p.mx_data = reinterpret_cast<uint16_t*>(mx_data_out);
  p.mx_scale = mx_scale_out;
  p.tp = tp;
  p.rows = rows;
  p.nv = hidden / 2;
  p.chunks = floor_chunks(hidden);
  hipLaunchKernelGGL(floor_boundary_kernel, dim3(floor_grid(rows, hidden)), dim3(kFloorBlock),
                     0, static_cast<hipStream_t>(stream), p);
  return hipGetLastError() == hipSuccess ? MHC_OK : MHC_ERR_HIP;
}

extern "C" int mhc_floor_empty(int rows, int hidden, mhc_stream_t stream) {
  if (!shape_ok(rows, hidden)) return MHC_ERR_SHAPE;
  if (rows == 0) return MHC_OK;
  FloorParams p = {};
  hipLaunchKernelGGL(floor_empty_kernel, dim3(floor_grid(rows, hidden)), dim3(kFloorBlock), 0,
                     static_cast<hipStream_t>(stream), p);
  return hipGetLastError() == hipSuccess ? MHC_OK : MHC_ERR_HIP;
}
