// The fused mHC boundary for gfx950: one memory-bound pass per call.
//
// Pages: boundary page (module docstring, Boundaries._reduce,
// Boundaries.post_only, empty_quantized_layer_input) and all_reduce page
// (BoundaryAllReduce.__call__ / finalize). The arithmetic of each step is
// stated in include/mhc.h.
//
// Work decomposition. A row (token) is split into `chunks` pieces of
// 8 * BS bf16 elements; one workgroup of BS threads owns one (row, chunk)
// and each thread one 16-byte vector of every tensor it touches, so every
// load and store is a coalesced 16-byte access. All of a thread's loads
// (tp partial slices, or top_k gathered expert rows plus the shared row, and
// the hc streams) are issued before the first use.
//
// The RMS of a row needs the whole row. Each workgroup writes its fp32
// collapse chunk y and its partial sum of y^2 to the handle's scratch,
// releases them, and bumps the row's arrival counter; the last workgroup to
// arrive for a row sums the partials in chunk order (deterministic, no float
// atomics), normalizes the whole row, writes the layer input and its MXFP8
// form, and returns the counter to zero for the next call.
//
// XCD placement. Consecutive workgroup ids are dealt round-robin to the 8
// XCDs, so a row's chunks are given ids congruent to the row mod 8: all
// workgroups of one row share one XCD's L2, where the scratch round trip
// stays.
#include "device_common.h"
#include "kernels.h"

namespace mhc {

constexpr int kHC = 4;
constexpr int kXcds = 8;

struct BoundaryParams {
  // sublayer output: TP partials ...
  const uint4* xp;          // [tp][rows][hv]
  int tp;
  // ... or an unfinalized MoE output
  const uint4* g;           // [num_permuted][hv]
  const float* ew;          // [rows][top_k]
  const int* idx;           // [rows * top_k]
  const uint4* shared;      // [rows][hv]
  int top_k, num_permuted;
  // mHC
  const uint4* res_in;      // [rows][4][hv]
  uint4* res_out;           // [rows][4][hv]
  const float* post;        // [rows][4]
  const float* comb;        // [rows][4][4]
  const float* pre;         // [rows][4]
  const uint4* norm_w;      // [hv]
  float eps;
  int rows, hv, hidden, chunks, rows_per_xcd;
  uint4* layer_out;         // [rows][hv]
  uint2* mx_data;           // [rows][hv] (8 E4M3 codes per vector)
  uint8_t* mx_scale;        // [rows][hidden / 32]
  // scratch
  float* ywork;             // [rows][hidden]
  float* part;              // [rows][max_chunks]
  unsigned* counters;       // [rows]
  int part_stride;
};

template <int BS, bool FINALIZE, bool HAS_PRE, bool MXFP8>
__global__ __launch_bounds__(BS) void boundary_kernel(const BoundaryParams p) {
  // --- (row, chunk) of this workgroup, XCD-aware -------------------------------
  const int wg = blockIdx.x;
  const int xcd = wg % kXcds;
  const int local = wg / kXcds;
  const int r = (local / p.chunks) * kXcds + xcd;
  const int c = local % p.chunks;
  if (r >= p.rows) return;  // padding workgroup (rows not a multiple of 8)

  const int tid = threadIdx.x;
  const int v = c * BS + tid;  // 16-byte vector index in the row
  const bool active = v < p.hv;

  // --- coefficients (uniform per workgroup) ------------------------------------
  float pst[kHC], cmb[kHC * kHC], pr[kHC];
#pragma unroll
  for (int i = 0; i < kHC; ++i) pst[i] = p.post[r * kHC + i];
#pragma unroll
  for (int i = 0; i < kHC * kHC; ++i) cmb[i] = p.comb[r * kHC * kHC + i];
  if constexpr (HAS_PRE) {
#pragma unroll
    for (int i = 0; i < kHC; ++i) pr[i] = p.pre[r * kHC + i];
  }

  float y[8];
  float sq = 0.f;
  if (active) {
    // --- loads: the sublayer output and the streams ----------------------------
    const uint4* res = p.res_in + (size_t)r * kHC * p.hv + v;
    uint4 sv[kHC];
#pragma unroll
    for (int j = 0; j < kHC; ++j) sv[j] = load_nt(res + (size_t)j * p.hv);

    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = 0.f;
    if constexpr (!FINALIZE) {
      const uint4* src = p.xp + (size_t)r * p.hv + v;
      const size_t slice = (size_t)p.rows * p.hv;
      for (int t0 = 0; t0 < p.tp; t0 += 8) {
        uint4 xv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (t0 + u < p.tp) xv[u] = load_nt(src + (size_t)(t0 + u) * slice);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (t0 + u < p.tp) {
            float f[8];
            unpack8(xv[u], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] += f[e];
          }
        }
      }
    } else {
      const uint4 shv = load_nt(p.shared + (size_t)r * p.hv + v);
      for (int k0 = 0; k0 < p.top_k; k0 += 8) {
        uint4 gv[8];
        float wk[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int k = k0 + u;
          wk[u] = 0.f;
          if (k < p.top_k) {
            const int pi = p.idx[r * p.top_k + k];
            if (pi >= 0 && pi < p.num_permuted) {
              wk[u] = p.ew[r * p.top_k + k];
              gv[u] = load_nt(p.g + (size_t)pi * p.hv + v);
            } else {
              gv[u] = make_uint4(0u, 0u, 0u, 0u);
            }
          }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (k0 + u < p.top_k) {
            float f[8];
            unpack8(gv[u], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = __builtin_fmaf(wk[u], f[e], x[e]);
          }
        }
      }
      float f[8];
      unpack8(shv, f);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] += f[e];
    }
    // the reduced output is a bf16 tensor
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = round_bf16(x[e]);

    // --- mHC post: s'_i = sum_j comb_ij s_j + post_i x ---------------------------
    float s[kHC][8];
#pragma unroll
    for (int j = 0; j < kHC; ++j) unpack8(sv[j], s[j]);
    uint4* out = p.res_out + (size_t)r * kHC * p.hv + v;
    float sn[kHC][8];
#pragma unroll
    for (int i = 0; i < kHC; ++i) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float a = pst[i] * x[e];
#pragma unroll
        for (int j = 0; j < kHC; ++j) a = __builtin_fmaf(cmb[i * kHC + j], s[j][e], a);
        sn[i][e] = a;
      }
      const uint4 o = pack8_round(sn[i]);
      out[(size_t)i * p.hv] = o;
      if constexpr (HAS_PRE) unpack8(o, sn[i]);  // the collapse reads the bf16 streams
    }

    // --- pre collapse and the chunk's sum of squares ------------------------------
    if constexpr (HAS_PRE) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float a = 0.f;
#pragma unroll
        for (int j = 0; j < kHC; ++j) a = __builtin_fmaf(pr[j], sn[j][e], a);
        y[e] = a;
        sq = __builtin_fmaf(a, a, sq);
      }
    }
  }
  if constexpr (!HAS_PRE) return;

  // --- publish the chunk: y to scratch, the partial sum of squares ---------------
  __shared__ float s_red[BS / kWave];
  __shared__ int s_last;
  __shared__ float s_inv;
  float* yrow = p.ywork + (size_t)r * p.hidden;
  if (active) {
    float4* dst = reinterpret_cast<float4*>(yrow + (size_t)v * 8);
    dst[0] = make_float4(y[0], y[1], y[2], y[3]);
    dst[1] = make_float4(y[4], y[5], y[6], y[7]);
  }
  sq = wave_sum(sq);
  if ((tid & (kWave - 1)) == 0) s_red[tid / kWave] = sq;
  __syncthreads();
  if (tid == 0) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < BS / kWave; ++w) t += s_red[w];
    p.part[(size_t)r * p.part_stride + c] = t;
  }
  __threadfence();  // release this thread's scratch stores at device scope
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = __hip_atomic_fetch_add(p.counters + r, 1u, __ATOMIC_ACQ_REL,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == (unsigned)(p.chunks - 1));
  }
  __syncthreads();
  if (!s_last) return;

  // --- last arriver: normalize the whole row ------------------------------------
  __threadfence();  // acquire: every chunk's scratch stores are visible
  if (tid == 0) {
    float tot = 0.f;
    for (int k = 0; k < p.chunks; ++k) tot += p.part[(size_t)r * p.part_stride + k];
    s_inv = 1.0f / sqrtf(tot / (float)p.hidden + p.eps);
    __hip_atomic_store(p.counters + r, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  const float inv = s_inv;
  for (int vv = tid; vv < p.hv; vv += BS) {
    const float4* src = reinterpret_cast<const float4*>(yrow + (size_t)vv * 8);
    const float4 a = src[0], b = src[1];
    float w[8];
    unpack8(p.norm_w[vv], w);
    float o[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (o[e] * inv) * w[e];
    const uint4 ob = pack8_round(o);
    p.layer_out[(size_t)r * p.hv + vv] = ob;
    if constexpr (MXFP8) {
      // 32-element block = the 4 consecutive lanes vv & ~3 .. vv | 3 (hidden % 32 == 0)
      float q[8];
      unpack8(ob, q);
      float amax = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(q[e]));
      amax = fmaxf(amax, __shfl_xor(amax, 1, kWave));
      amax = fmaxf(amax, __shfl_xor(amax, 2, kWave));
      const int ex = e8m0_exponent(__float_as_uint(amax));
      const float sc = __uint_as_float((uint32_t)(127 - ex) << 23);  // 2^-e, exact
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) lo |= f32_to_e4m3(q[e] * sc) << (8 * e);
#pragma unroll
      for (int e = 0; e < 4; ++e) hi |= f32_to_e4m3(q[4 + e] * sc) << (8 * e);
      p.mx_data[(size_t)r * p.hv + vv] = make_uint2(lo, hi);
      if ((vv & 3) == 0) p.mx_scale[(size_t)r * (p.hidden / 32) + (vv >> 2)] = (uint8_t)(ex + 127);
    }
  }
}

// ---------------------------------------------------------------------------
// mean over the hc streams: out[r,h] = bf16( (1/4) sum_i s[r,i,h] )
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void collapse_mean_kernel(const uint4* __restrict__ s,
                                                            uint4* __restrict__ out, int rows,
                                                            int hv) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)rows * hv) return;
  const int r = (int)(i / hv), v = (int)(i % hv);
  const uint4* src = s + (size_t)r * kHC * hv + v;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  uint4 sv[kHC];
#pragma unroll
  for (int j = 0; j < kHC; ++j) sv[j] = load_nt(src + (size_t)j * hv);
#pragma unroll
  for (int j = 0; j < kHC; ++j) {
    float f[8];
    unpack8(sv[j], f);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += f[e];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] *= 0.25f;
  out[i] = pack8_round(acc);
}

// ---------------------------------------------------------------------------
// host-side launchers
// ---------------------------------------------------------------------------
template <int BS, bool FIN, bool PRE, bool MX>
static hipError_t launch_one(const BoundaryParams& p, int grid, hipStream_t st) {
  hipLaunchKernelGGL((boundary_kernel<BS, FIN, PRE, MX>), dim3(grid), dim3(BS), 0, st, p);
  return hipGetLastError();
}

template <int BS>
static hipError_t launch_bs(const BoundaryParams& p, bool fin, bool pre, bool mx, int grid,
                            hipStream_t st) {
  if (!fin) {
    if (!pre) return launch_one<BS, false, false, false>(p, grid, st);
    return mx ? launch_one<BS, false, true, true>(p, grid, st)
              : launch_one<BS, false, true, false>(p, grid, st);
  }
  if (!pre) return launch_one<BS, true, false, false>(p, grid, st);
  return mx ? launch_one<BS, true, true, true>(p, grid, st)
            : launch_one<BS, true, true, false>(p, grid, st);
}

int boundary_chunks(int hidden, int block) {
  const int hv = hidden / 8;
  return (hv + block - 1) / block;
}

hipError_t launch_boundary(const BoundaryLaunch& L, hipStream_t stream) {
  BoundaryParams p;
  p.xp = reinterpret_cast<const uint4*>(L.x_partials);
  p.tp = L.tp;
  p.g = reinterpret_cast<const uint4*>(L.gemm2_permuted);
  p.ew = L.expert_weights;
  p.idx = L.idx;
  p.shared = reinterpret_cast<const uint4*>(L.shared_output);
  p.top_k = L.top_k;
  p.num_permuted = L.num_permuted;
  p.res_in = reinterpret_cast<const uint4*>(L.residual);
  p.res_out = reinterpret_cast<uint4*>(L.residual_out);
  p.post = L.post;
  p.comb = L.comb;
  p.pre = L.pre;
  p.norm_w = reinterpret_cast<const uint4*>(L.norm_weight);
  p.eps = L.eps;
  p.rows = L.rows;
  p.hidden = L.hidden;
  p.hv = L.hidden / 8;
  p.chunks = boundary_chunks(L.hidden, L.block);
  p.layer_out = reinterpret_cast<uint4*>(L.layer_input_out);
  p.mx_data = reinterpret_cast<uint2*>(L.mx_data_out);
  p.mx_scale = L.mx_scale_out;
  p.ywork = L.ywork;
  p.part = L.part;
  p.counters = L.counters;
  p.part_stride = L.part_stride;
  p.rows_per_xcd = (L.rows + kXcds - 1) / kXcds;
  const int grid = kXcds * p.rows_per_xcd * p.chunks;
  const bool fin = L.gemm2_permuted != nullptr;
  const bool pre = L.pre != nullptr;
  const bool mx = L.mx_data_out != nullptr;
  switch (L.block) {
    case 64: return launch_bs<64>(p, fin, pre, mx, grid, stream);
    case 128: return launch_bs<128>(p, fin, pre, mx, grid, stream);
    case 256: return launch_bs<256>(p, fin, pre, mx, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_collapse_mean(const uint16_t* streams, int rows, int hidden, uint16_t* out,
                                hipStream_t stream) {
  const int hv = hidden / 8;
  const long long n = (long long)rows * hv;
  const int grid = (int)((n + 255) / 256);
  hipLaunchKernelGGL(collapse_mean_kernel, dim3(grid), dim3(256), 0, stream,
                     reinterpret_cast<const uint4*>(streams), reinterpret_cast<uint4*>(out), rows,
                     hv);
  return hipGetLastError();
}

}  // namespace mhc
