// The coefficient epilogue of one row, run by one full wave: the split-K partial sums of
// the fn projection and of sum v^2 are added in split order, then 1/RMS, scale and base,
// the sigmoids of pre and post, and the Sinkhorn iterations of comb.
//
// Pages: boundary page, Boundaries.sublayer and Boundaries._pre (the coefficient call's
// arguments); the arithmetic is stated in include/mhc.h (mhc_pre_coeffs).
//
// Shared by the coefficient path's own epilogue kernel and by the boundary kernels that
// finish a deferred coefficient call, so both produce the same bits.
#pragma once

#include "device_common.h"

namespace mhc {

constexpr int kCoefN = 4;                            // hc_mult
constexpr int kCoefNC = 2 * kCoefN + kCoefN * kCoefN;  // 24 logits
constexpr int kCoefPartW = kCoefNC + 1;              // + sum of squares

struct CoeffEpilogue {
  const float* part;     // [rows_pad][ks_count / 4][25][4] split-K partials (coeff_part_index)
  const float* scale;    // [3]
  const float* base;     // [24]
  int ks_count;          // a multiple of 4
  int K;                 // n * hidden
  float rms_eps, pre_eps, sk_eps, alpha;
  int iters;
};

// This lane's scale and base (lanes >= 24 read entry 23; their value is unused).
__device__ __forceinline__ void coeff_lane_scale_base(const CoeffEpilogue& e, int L, float* sc,
                                                      float* bs) {
  const int Lc = L < kCoefNC ? L : kCoefNC - 1;
  *sc = e.scale[Lc < kCoefN ? 0 : (Lc < 2 * kCoefN ? 1 : 2)];
  *bs = e.base[Lc];
}

// The first splits of a lane's partials, fetched ahead so that their latency overlaps
// other work: NP x 4 splits (NP x 16 bytes per lane).
template <int NP>
struct CoeffPrefetch {
  float4 v[NP];
};

// The split-K partials of a row: value L (logit L < 24, the sum of squares at 24) of split s
// sits at coeff_part_index(r, L, s, ks): per row, one float4 of four consecutive splits per
// value, the 25 values of a split quad contiguous. A reader lane of value L then loads its
// splits four at a time, and the lanes of a row read one contiguous 400-byte block per quad.
__host__ __device__ __forceinline__ size_t coeff_part_index(int r, int L, int s, int ks) {
  return (((size_t)r * (ks / 4) + s / 4) * kCoefPartW + L) * 4 + (s & 3);
}

// Value L's splits 4u .. 4u + 3 of row r (the partials are far below 4 GiB: a 32-bit
// byte offset).
__device__ __forceinline__ float4 coeff_quad(const CoeffEpilogue& e, int r, int L, int u) {
  const uint32_t off = ((((uint32_t)r * (uint32_t)(e.ks_count / 4) + (uint32_t)u) * kCoefPartW +
                         (uint32_t)L) * 16u);
  return *byte_at(reinterpret_cast<const float4*>(e.part), off);
}

// Lanes 0..24 (logits 0..23 and the sum of squares) load their first splits of row r.
// With ALL_LANES the other lanes load lane 24's too (so that no load sits behind a
// lane-dependent branch, for callers that have other loads in flight); their sums go
// unused.
template <bool ALL_LANES, int NP>
__device__ __forceinline__ void coeff_row_prefetch(const CoeffEpilogue& e, int r, int L,
                                                   CoeffPrefetch<NP>& f) {
  if (!ALL_LANES && L >= kCoefPartW) return;
  const int Lc = L < kCoefPartW ? L : kCoefPartW - 1;
  const int last = e.ks_count / 4 - 1;  // past it: in-bounds repeats, never added
#pragma unroll
  for (int u = 0; u < NP; ++u) f.v[u] = coeff_quad(e, r, Lc, u < last ? u : last);
}

__device__ __forceinline__ float coeff_from_sums(const CoeffEpilogue& e, int L, float acc,
                                                 float sc_l, float base_l, int* slot);

// Row r's coefficients after coeff_row_prefetch; every lane of the wave must call it
// (lane = L). Returns this lane's value and sets *slot: 0..3 pre, 4..7 post, 8..23 comb
// (row-major), -1 none.
template <bool ALL_LANES, int NP>
__device__ __forceinline__ float coeff_row_finish(const CoeffEpilogue& e, int r, int L,
                                                  const CoeffPrefetch<NP>& f, float sc_l,
                                                  float base_l, int* slot) {
  // each lane adds its splits in split order: the prefetched ones, then the rest in
  // batches that are fetched whole before they are added
  float acc = 0.f;
  if (ALL_LANES || L < kCoefPartW) {
    const int n4 = e.ks_count / 4;
#pragma unroll
    for (int u = 0; u < NP; ++u)
      if (u < n4) acc = (((acc + f.v[u].x) + f.v[u].y) + f.v[u].z) + f.v[u].w;
    const int Lc = L < kCoefPartW ? L : kCoefPartW - 1;
    constexpr int kBatch = 16;
    for (int b0 = NP; b0 < n4; b0 += kBatch) {  // splits beyond the prefetched ones
      float4 v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int i = b0 + u;
        v[u] = coeff_quad(e, r, Lc, i < n4 ? i : n4 - 1);  // in-bounds repeats, never added
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (b0 + u < n4) acc = (((acc + v[u].x) + v[u].y) + v[u].z) + v[u].w;
    }
  }
  return coeff_from_sums(e, L, acc, sc_l, base_l, slot);
}

// Row coefficients from this lane's complete sum (lane L < 24: logit L, lane 24: the sum
// of squares, others unused); every lane of the wave must call it. Returns this lane's
// value and sets *slot as coeff_row_finish.
__device__ __forceinline__ float coeff_from_sums(const CoeffEpilogue& e, int L, float acc,
                                                 float sc_l, float base_l, int* slot) {
  const float ss = __shfl(acc, kCoefNC, kWave);
  const float inv = fast_rsq(ss * fast_rcp((float)e.K) + e.rms_eps);
  float lp = 0.f;
  if (L < kCoefNC) lp = (acc * inv) * sc_l + base_l;
  float out = 0.f;
  *slot = -1;
  if (L < kCoefN) {
    out = fast_rcp(1.0f + fast_exp(-lp)) + e.pre_eps;
    *slot = L;
  } else if (L < 2 * kCoefN) {
    out = e.alpha * fast_rcp(1.0f + fast_exp(-lp));
    *slot = L;
  }
  // comb: the 16 entries sit in lanes 32..47 (one DPP row), entry (i, j) at lane 32 + 4i + j,
  // so a row sum is two quad steps and a column sum two row rotations. Every lane runs the
  // same instructions (lanes outside the row carry dummies).
  const int ce = L - 32;  // entry index for lanes 32..47
  float a = __shfl(lp, 2 * kCoefN + (ce & 15), kWave);
  float mx = fmaxf(a, dpp_f32<kDppQuadXor1>(a));
  mx = fmaxf(mx, dpp_f32<kDppQuadXor2>(mx));
  a = fast_exp(a - mx);
  for (int it = 0; it < e.iters; ++it) {
    float rs = a + dpp_f32<kDppQuadXor1>(a);
    rs = rs + dpp_f32<kDppQuadXor2>(rs);
    a = a * __builtin_amdgcn_rcpf(rs + e.sk_eps);
    float cs = a + dpp_f32<kDppRowRor4>(a);
    cs = cs + dpp_f32<kDppRowRor8>(cs);
    a = a * __builtin_amdgcn_rcpf(cs + e.sk_eps);
  }
  if (ce >= 0 && ce < kCoefN * kCoefN) {
    out = a;
    *slot = 2 * kCoefN + ce;
  }
  return out;
}

// Both phases back to back, loads on lanes 0..24 only, up to 64 splits in one batch.
__device__ __forceinline__ float coeff_row(const CoeffEpilogue& e, int r, int L, float sc_l,
                                           float base_l, int* slot) {
  CoeffPrefetch<16> f;
  coeff_row_prefetch<false>(e, r, L, f);
  return coeff_row_finish<false>(e, r, L, f, sc_l, base_l, slot);
}

}  // namespace mhc
