// The mHC coefficient path for gfx950: flattened RMS, fn projection on MFMA,
// scale/base, sigmoid pre/post and the Sinkhorn-normalized comb.
//
// Pages: boundary page, Boundaries.sublayer and Boundaries._pre (the
// coefficient call's arguments); the arithmetic is stated in include/mhc.h.
//
// Kernel 1 (split-K): the projection l[r,c] = sum_k v[r,k] fn[k,c] is a skinny
// GEMM (M = rows, N = 24 logits, K = n*hidden). Each workgroup owns 16 rows and
// one contiguous range of 32-wide k steps; its four waves take alternate steps
// and run v_mfma_f32_16x16x32_bf16 on the raw bf16 operands (bf16 products are
// exact in fp32, and 1/RMS is applied afterwards, so no normalized copy is
// rounded). The MFMA's M side is fn^T (logit columns 0..15 and 16..31, the
// last 8 zero), its N side is the 16 rows. The same pass accumulates the
// rows' sums of squares. Partials go to scratch [k-split][row][25].
//
// Kernel 2: one wave per row sums the k-split partials in a fixed order, then
// applies 1/RMS, scale/base, the sigmoids and the Sinkhorn iterations, one lane
// per logit (the 16 comb entries sit in lanes 32..47, row i / column j at lane
// 32 + 4i + j, so row sums are quad butterflies and column sums use xor 4, 8).
#include "device_common.h"
#include "kernels.h"

namespace mhc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kN = 4;                      // hc_mult
constexpr int kNC = 2 * kN + kN * kN;      // 24 logits
constexpr int kPartW = kNC + 1;            // + sum of squares
constexpr int kRB = 16;                    // rows per workgroup (MFMA N)
constexpr int kStepK = 32;                 // MFMA K
constexpr int kPreWaves = 4;

struct PrePartialParams {
  const uint16_t* res;   // [rows][K] bf16 (the streams, flattened)
  const uint16_t* fn;    // [K][24] bf16
  float* part;           // [ks][rows_pad][25]
  int rows, K, ks_count, steps_per_wg, nsteps, rows_pad;
};

__global__ __launch_bounds__(kPreWaves * kWave) void pre_partial_kernel(const PrePartialParams p) {
  const int wg = blockIdx.x;
  const int ks = wg % p.ks_count;  // ks_count % 8 == 0: a k range stays on one XCD
  const int rb = wg / p.ks_count;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int m = lane & 15;   // MFMA row of A (logit column) / column of B (row)
  const int kg = lane >> 4;  // which 8 of the 32 k
  const int row = rb * kRB + m;
  const bool row_ok = row < p.rows;
  const bool c1_ok = (16 + m) < kNC;

  const int s0 = ks * p.steps_per_wg;
  const int s1 = min(s0 + p.steps_per_wg, p.nsteps);

  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  float sq = 0.f;
  const uint16_t* vrow = p.res + (size_t)(row_ok ? row : 0) * p.K;
  for (int s = s0 + wave; s < s1; s += kPreWaves) {
    const int k0 = s * kStepK + kg * 8;
    uint4 bv = make_uint4(0u, 0u, 0u, 0u);
    if (row_ok) bv = load_nt(reinterpret_cast<const uint4*>(vrow + k0));
    short8_t a0, a1;
    const uint16_t* f = p.fn + (size_t)k0 * kNC;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      a0[j] = (short)f[j * kNC + m];
      a1[j] = c1_ok ? (short)f[j * kNC + 16 + m] : (short)0;
    }
    const bf16x8_t b = __builtin_bit_cast(bf16x8_t, bv);
    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a0), b, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a1), b, acc1, 0, 0, 0);
    float x[8];
    unpack8(bv, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) sq = __builtin_fmaf(x[e], x[e], sq);
  }
  // the four k groups of a row -> lanes m
  sq += __shfl_xor(sq, 16, kWave);
  sq += __shfl_xor(sq, 32, kWave);

  __shared__ float red[kPreWaves][kRB][kPartW];
  // D layout: lane holds D[4*(lane/16) + i][lane % 16]: logit column 4*kg + i (+16), row m
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    red[wave][m][4 * kg + i] = acc0[i];
    if (kg < 2) red[wave][m][16 + 4 * kg + i] = acc1[i];
  }
  if (kg == 0) red[wave][m][kNC] = sq;
  __syncthreads();
  for (int o = tid; o < kRB * kPartW; o += kPreWaves * kWave) {
    const int rr = o / kPartW, cc = o % kPartW;
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kPreWaves; ++w) t += red[w][rr][cc];
    p.part[((size_t)ks * p.rows_pad + rb * kRB + rr) * kPartW + cc] = t;
  }
}

struct PreEpilogueParams {
  const float* part;
  const float* scale;  // [3]
  const float* base;   // [24]
  float* pre_out;      // [rows][4]
  float* post_out;     // [rows][4]
  float* comb_out;     // [rows][16]
  float rms_eps, pre_eps, sk_eps, alpha;
  int iters, rows, K, ks_count, rows_pad;
};

__global__ __launch_bounds__(kWave) void pre_epilogue_kernel(const PreEpilogueParams p) {
  const int r = blockIdx.x;
  const int L = threadIdx.x;
  int col = -1;
  if (L < 2 * kN) col = L;
  else if (L >= 32 && L < 32 + kN * kN) col = 2 * kN + (L - 32);
  else if (L == kWave - 1) col = kNC;  // sum of squares

  float acc = 0.f;
  if (col >= 0) {
    const float* src = p.part + (size_t)r * kPartW + col;
    const size_t stride = (size_t)p.rows_pad * kPartW;
    for (int k = 0; k < p.ks_count; ++k) acc += src[(size_t)k * stride];
  }
  const float ss = __shfl(acc, kWave - 1, kWave);
  const float inv = 1.0f / sqrtf(ss / (float)p.K + p.rms_eps);
  float lp = 0.f;
  if (col >= 0 && col < kNC) {
    const int g = col < kN ? 0 : (col < 2 * kN ? 1 : 2);
    lp = (acc * inv) * p.scale[g] + p.base[col];
  }
  if (L < kN) {
    p.pre_out[r * kN + L] = 1.0f / (1.0f + expf(-lp)) + p.pre_eps;
  } else if (L < 2 * kN) {
    p.post_out[r * kN + (L - kN)] = p.alpha * (1.0f / (1.0f + expf(-lp)));
  }
  // Sinkhorn over lanes 32..47 (every lane runs the shuffles; others carry dummies)
  float mx = fmaxf(lp, __shfl_xor(lp, 1, kWave));
  mx = fmaxf(mx, __shfl_xor(mx, 2, kWave));
  float a = expf(lp - mx);
  for (int it = 0; it < p.iters; ++it) {
    float rs = a + __shfl_xor(a, 1, kWave);
    rs = rs + __shfl_xor(rs, 2, kWave);
    a = a / (rs + p.sk_eps);
    float cs = a + __shfl_xor(a, 4, kWave);
    cs = cs + __shfl_xor(cs, 8, kWave);
    a = a / (cs + p.sk_eps);
  }
  if (L >= 32 && L < 32 + kN * kN) p.comb_out[r * kN * kN + (L - 32)] = a;
}

void pre_plan(int rows, int hidden, int* ks_count, int* steps_per_wg, int* rows_pad) {
  const int K = kN * hidden;
  const int nsteps = K / kStepK;
  const int rbn = (rows + kRB - 1) / kRB;
  int ks = (512 / rbn) / 8 * 8;
  const int cap = (nsteps / kPreWaves) / 8 * 8;
  if (ks > cap) ks = cap;
  if (ks > 256) ks = 256;
  if (ks < 8) ks = 8;
  *ks_count = ks;
  *steps_per_wg = (nsteps + ks - 1) / ks;
  *rows_pad = rbn * kRB;
}

size_t pre_scratch_floats_for(int rows, int hidden) {
  int ks, spw, rp;
  pre_plan(rows, hidden, &ks, &spw, &rp);
  return (size_t)ks * rp * kPartW;
}

hipError_t launch_pre_coeffs(const PreLaunch& L, hipStream_t stream) {
  int ks, spw, rp;
  pre_plan(L.rows, L.hidden, &ks, &spw, &rp);
  PrePartialParams a;
  a.res = L.residual;
  a.fn = L.fn;
  a.part = L.part;
  a.rows = L.rows;
  a.K = kN * L.hidden;
  a.ks_count = ks;
  a.steps_per_wg = spw;
  a.nsteps = a.K / kStepK;
  a.rows_pad = rp;
  const int grid = ks * (rp / kRB);
  hipLaunchKernelGGL(pre_partial_kernel, dim3(grid), dim3(kPreWaves * kWave), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  PreEpilogueParams b;
  b.part = L.part;
  b.scale = L.scale;
  b.base = L.base;
  b.pre_out = L.pre_out;
  b.post_out = L.post_out;
  b.comb_out = L.comb_out;
  b.rms_eps = L.rms_eps;
  b.pre_eps = L.pre_eps;
  b.sk_eps = L.sinkhorn_eps;
  b.alpha = L.post_alpha;
  b.iters = L.sinkhorn_iters;
  b.rows = L.rows;
  b.K = a.K;
  b.ks_count = ks;
  b.rows_pad = rp;
  hipLaunchKernelGGL(pre_epilogue_kernel, dim3(L.rows), dim3(kWave), 0, stream, b);
  return hipGetLastError();
}

}  // namespace mhc
