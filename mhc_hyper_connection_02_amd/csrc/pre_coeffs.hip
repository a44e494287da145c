// The mHC coefficient path for gfx950: flattened RMS, fn projection on MFMA,
// scale/base, sigmoid pre/post and the Sinkhorn-normalized comb.
//
// Pages: boundary page, Boundaries.sublayer and Boundaries._pre (the
// coefficient call's arguments); the arithmetic is stated in include/mhc.h.
//
// Kernel 1 (split-K): the projection l[r,c] = sum_k v[r,k] fn[k,c] is a skinny
// GEMM (M = rows, N = 24 logits, K = n*hidden), HBM-bound. Each workgroup owns
// 16 rows and one contiguous range of 32-wide k steps. It first copies its
// slice of fn (contiguous in memory: [k range][24]) into LDS with 16-byte
// loads, transposed to [logit][k] so that each lane's MFMA operand (8
// consecutive k of one logit column) is one 16-byte LDS read. Its four waves
// then take alternate k steps and run v_mfma_f32_16x16x32_bf16 on the raw
// bf16 operands (bf16 products are exact in fp32; 1/RMS is applied
// afterwards, so no normalized copy is rounded). The MFMA's M side is fn^T
// (logit columns 0..15 and 16..31, the last 8 zero), its N side the 16 rows.
// The same pass accumulates the rows' sums of squares. Each workgroup writes
// its 16 x 25 partials to scratch laid out per row by quads of k-splits
// (coeff_part_index), so that the epilogue's lanes, one per logit, read
// contiguous blocks four splits at a time.
//
// Kernel 2: one wave per row runs the row's epilogue (coeff_epilogue.h): the
// k-split partials added in split order, 1/RMS, scale and base, the sigmoids
// and the Sinkhorn iterations. A deferred call (mhc_pre_coeffs_deferred)
// launches only kernel 1 and leaves kernel 2's work to the boundary kernel
// that consumes the coefficients, which runs the same function.
#include "coeff_epilogue.h"
#include "device_common.h"
#include "kernels.h"

namespace mhc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kN = 4;                      // hc_mult
constexpr int kNC = 2 * kN + kN * kN;      // 24 logits
constexpr int kPartW = kNC + 1;            // + sum of squares
constexpr int kRB = 16;                    // rows per workgroup (MFMA N)
constexpr int kStepK = 32;                 // MFMA K
constexpr int kPreWaves = 4;
constexpr int kTargetWgs = 256;
constexpr int kMaxStepsPerWg = 32;         // LDS: 24 x (32*32 + 8) bf16 = 49.5 KB
constexpr int kLdsPad = 8;

struct PrePartialParams {
  const uint16_t* res;   // [rows][K] bf16 (the streams, flattened)
  const uint16_t* fn;    // [K][24] bf16
  float* part;           // [rows_pad][ks / 4][25][4] (coeff_part_index)
  int rows, K, ks_count, steps_per_wg, nsteps;
};

// NS: the k steps a wave owns (ceil(steps per workgroup / 4), 1..8), so that the number of
// loads is known at compile time and every load can be unconditional.
template <int NS>
__global__ __launch_bounds__(kPreWaves * kWave) void pre_partial_kernel(const PrePartialParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t fnT[kNC][kMaxStepsPerWg * kStepK + kLdsPad];
  __shared__ float red[kPreWaves][kRB][kPartW];
  static_assert(NS >= 1 && NS * kPreWaves <= kMaxStepsPerWg, "steps per wave");
  constexpr int kMaxWaveSteps = NS;
  // the slice's fn vectors (NS * 4 steps of 32 k, 3 vectors a k row) over the threads
  constexpr int kMaxFnVecs = (NS * kPreWaves * kStepK * kNC / 8 + kPreWaves * kWave - 1) /
                             (kPreWaves * kWave);

  const int wg = blockIdx.x;
  // (row block, split) pairs are dealt to the 8 XCDs in contiguous ranges (the grid,
  // row blocks x ks_count, is a multiple of 8): the splits of a (row, logit), adjacent in
  // `part`, are then written from one XCD's L2 (0.9 us less per 128-row call than dealing
  // consecutive splits to consecutive XCDs; the same at 64 rows)
  const int idx = (wg % 8) * ((int)gridDim.x / 8) + wg / 8;
  const int ks = idx % p.ks_count;
  const int rb = idx / p.ks_count;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int m = lane & 15;   // MFMA row of A (logit column) / column of B (row)
  const int kg = lane >> 4;  // which 8 of the 32 k
  const int row = rb * kRB + m;
  const bool row_ok = row < p.rows;

  const int s0 = ks * p.steps_per_wg;
  const int s1 = min(s0 + p.steps_per_wg, p.nsteps);
  const int kbase = s0 * kStepK;

  // --- every load first: the fn slice (its staging into LDS then waits for it alone), then
  // this wave's row vectors (steps s0 + wave + 4i). Every load is unconditional, its index
  // clamped into the tensor (rows past the last read row 0, steps and vectors past the slice
  // the tensor's last ones): those values are never used (steps, vectors) or only reach
  // rows that are never read. A load behind a branch (a zero for the missing rows, a bound
  // on the steps or vectors) made the compiler wait for it, or for every load, before going
  // on.
  const uint4* src = reinterpret_cast<const uint4*>(p.fn);
  const int last_vec = p.nsteps * kStepK * kNC / 8 - 1;
  uint4 fv[kMaxFnVecs];
#pragma unroll
  for (int j = 0; j < kMaxFnVecs; ++j) {
    const int i = tid + j * kPreWaves * kWave;
    fv[j] = src[min(kbase * kNC / 8 + i, last_vec)];
  }
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint16_t* vrow = p.res + (size_t)(row_ok ? row : 0) * p.K + kg * 8;
  uint4 bv[kMaxWaveSteps];
#pragma unroll
  for (int i = 0; i < kMaxWaveSteps; ++i) {
    const int gs = min(s0 + wave_u + kPreWaves * i, p.nsteps - 1);  // global step
    bv[i] = load_nt(reinterpret_cast<const uint4*>(vrow + gs * kStepK));
  }
  // --- fn slice -> LDS, transposed to [logit][k]; every lane writes (past the slice, at
  // k past the workgroup's steps inside the buffer, which no MFMA step reads)
#pragma unroll
  for (int j = 0; j < kMaxFnVecs; ++j) {
    const int i = tid + j * kPreWaves * kWave;
    const int e = i * 8;
    const int kk = e / kNC, c0 = e % kNC;  // c0 in {0, 8, 16}; kk < kMaxStepsPerWg * kStepK
    const uint32_t u[4] = {fv[j].x, fv[j].y, fv[j].z, fv[j].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      fnT[c0 + 2 * q][kk] = (uint16_t)(u[q] & 0xFFFFu);
      fnT[c0 + 2 * q + 1][kk] = (uint16_t)(u[q] >> 16);
    }
  }
  __syncthreads();

  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  float sq = 0.f;
  // logits 16..31, of which 24..31 are zero: the load reads a row that exists and the value
  // is masked, so it stays an LDS read (a select between the LDS row and a zero in a local
  // variable compiled to a generic load from either place, with a wait for every
  // outstanding memory access)
  const bool hi_ok = 16 + m < kNC;
  const uint32_t keep = hi_ok ? ~0u : 0u;
#pragma unroll
  for (int i = 0; i < kMaxWaveSteps; ++i) {
    const int sl = wave_u + kPreWaves * i;
    if (s0 + sl < s1) {
      const int kl = sl * kStepK + kg * 8;  // k offset inside the slice
      const uint4 a0 = *reinterpret_cast<const uint4*>(&fnT[m][kl]);
      uint4 a1 = *reinterpret_cast<const uint4*>(&fnT[hi_ok ? 16 + m : m][kl]);
      a1.x &= keep;
      a1.y &= keep;
      a1.z &= keep;
      a1.w &= keep;
      const bf16x8_t b = __builtin_bit_cast(bf16x8_t, bv[i]);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a0), b, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a1), b, acc1, 0, 0, 0);
      float x[8];
      unpack8(bv[i], x);
#pragma unroll
      for (int e = 0; e < 8; ++e) sq = __builtin_fmaf(x[e], x[e], sq);
    }
  }
  // the four k groups of a row -> lanes m
  sq += __shfl_xor(sq, 16, kWave);
  sq += __shfl_xor(sq, 32, kWave);

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
    p.part[coeff_part_index(rb * kRB + rr, cc, ks, p.ks_count)] = t;
  }
}

struct PreEpilogueParams {
  CoeffEpilogue e;
  float* pre_out;      // [rows][4]
  float* post_out;     // [rows][4]
  float* comb_out;     // [rows][16]
};

__global__ __launch_bounds__(kWave) void pre_epilogue_kernel(const PreEpilogueParams p) {
  // rows dealt to the 8 XCDs in contiguous ranges (when the row count allows): XCD x then
  // finishes the rows whose partials the split-K kernel wrote from XCD x at 128 rows (read
  // from its own L2), and its outputs do not share lines with other XCDs' (measured 0.4 us
  // less per 128-row call; the same at 64 rows)
  const int nb = (int)gridDim.x;
  const int r = (nb % 8 == 0) ? ((int)blockIdx.x % 8) * (nb / 8) + (int)blockIdx.x / 8
                              : (int)blockIdx.x;
  const int L = threadIdx.x;
  float sc_l, base_l;
  coeff_lane_scale_base(p.e, L, &sc_l, &base_l);  // early: they arrive with the partials
  int slot;
  const float v = coeff_row(p.e, r, L, sc_l, base_l, &slot);
  if (slot >= 0 && slot < kN) p.pre_out[r * kN + slot] = v;
  else if (slot >= kN && slot < 2 * kN) p.post_out[r * kN + slot - kN] = v;
  else if (slot >= 2 * kN) p.comb_out[r * kN * kN + slot - 2 * kN] = v;
}

void pre_plan(int rows, int hidden, int* ks_count, int* steps_per_wg, int* rows_pad) {
  const int K = kN * hidden;
  const int nsteps = K / kStepK;
  const int rbn = (rows + kRB - 1) / kRB;
  int ks = (kTargetWgs / rbn) / 8 * 8;
  if (ks < 8) ks = 8;
  // every workgroup's slice must fit the LDS staging buffer
  const int min_ks = (nsteps + kMaxStepsPerWg - 1) / kMaxStepsPerWg;
  if (ks < min_ks) ks = (min_ks + 7) / 8 * 8;
  int spw = (nsteps + ks - 1) / ks;
  if (spw < 1) spw = 1;
  *ks_count = ks;
  *steps_per_wg = spw;
  *rows_pad = rbn * kRB;
}

size_t pre_scratch_floats_for(int rows, int hidden) {
  int ks, spw, rp;
  pre_plan(rows, hidden, &ks, &spw, &rp);
  return (size_t)ks * rp * kPartW;
}

CoeffEpilogue pre_epilogue_args(const PreLaunch& L) {
  int ks, spw, rp;
  pre_plan(L.rows, L.hidden, &ks, &spw, &rp);
  CoeffEpilogue e;
  e.part = L.part;
  e.scale = L.scale;
  e.base = L.base;
  e.ks_count = L.ks_count > 0 ? L.ks_count : ks;
  e.K = kN * L.hidden;
  e.rms_eps = L.rms_eps;
  e.pre_eps = L.pre_eps;
  e.sk_eps = L.sinkhorn_eps;
  e.alpha = L.post_alpha;
  e.iters = L.sinkhorn_iters;
  return e;
}

hipError_t launch_pre_partial(const PreLaunch& L, hipStream_t stream) {
  int ks, spw, rp;
  pre_plan(L.rows, L.hidden, &ks, &spw, &rp);
  if (spw > kMaxStepsPerWg) return hipErrorInvalidConfiguration;
  PrePartialParams a;
  a.res = L.residual;
  a.fn = L.fn;
  a.part = L.part;
  a.rows = L.rows;
  a.K = kN * L.hidden;
  a.ks_count = ks;
  a.steps_per_wg = spw;
  a.nsteps = a.K / kStepK;
  const int grid = ks * (rp / kRB);
  const dim3 g(grid), b(kPreWaves * kWave);
  switch ((spw + kPreWaves - 1) / kPreWaves) {
    case 1: hipLaunchKernelGGL(pre_partial_kernel<1>, g, b, 0, stream, a); break;
    case 2: hipLaunchKernelGGL(pre_partial_kernel<2>, g, b, 0, stream, a); break;
    case 3: hipLaunchKernelGGL(pre_partial_kernel<3>, g, b, 0, stream, a); break;
    case 4: hipLaunchKernelGGL(pre_partial_kernel<4>, g, b, 0, stream, a); break;
    case 5: hipLaunchKernelGGL(pre_partial_kernel<5>, g, b, 0, stream, a); break;
    case 6: hipLaunchKernelGGL(pre_partial_kernel<6>, g, b, 0, stream, a); break;
    case 7: hipLaunchKernelGGL(pre_partial_kernel<7>, g, b, 0, stream, a); break;
    case 8: hipLaunchKernelGGL(pre_partial_kernel<8>, g, b, 0, stream, a); break;
    default: return hipErrorInvalidConfiguration;
  }
  return hipGetLastError();
}

hipError_t launch_pre_epilogue(const PreLaunch& L, hipStream_t stream) {
  PreEpilogueParams b;
  b.e = pre_epilogue_args(L);
  b.pre_out = L.pre_out;
  b.post_out = L.post_out;
  b.comb_out = L.comb_out;
  hipLaunchKernelGGL(pre_epilogue_kernel, dim3(L.rows), dim3(kWave), 0, stream, b);
  return hipGetLastError();
}

hipError_t launch_pre_coeffs(const PreLaunch& L, hipStream_t stream) {
  hipError_t e = launch_pre_partial(L, stream);
  if (e != hipSuccess) return e;
  return launch_pre_epilogue(L, stream);
}

}  // namespace mhc
