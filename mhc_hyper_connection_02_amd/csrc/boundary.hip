// The fused mHC boundary for gfx950: one memory-bound pass per call.
//
// Pages: boundary page (module docstring, Boundaries._reduce,
// Boundaries.post_only, empty_quantized_layer_input) and all_reduce page
// (BoundaryAllReduce.__call__ / finalize). The arithmetic of each step is
// stated in include/mhc.h.
//
// Work decomposition. A row (token) is split into `chunks` pieces; one
// workgroup of BS threads owns one (row, chunk), one lane per vector of EL
// consecutive hidden elements (EL = 8, 4 or 2: a 16-, 8- or 4-byte vector; BS
// vectors per workgroup). The lane loads the vector's partial slices (or
// gathered expert rows) and its four streams and computes the four new
// streams; the kernels that write a layer input also load its norm weights and
// compute the collapse and its share of the row's sum of squares. The
// residual-only kernels run at two elements per lane and 512 threads.
// A lane issues all of its loads before the first use and stores its new
// streams as soon as they are computed; only the layer input (and its MXFP8
// form) waits for the row's RMS.
//
// The row RMS. The RMS needs the whole row, and a row spans several
// workgroups. Every wave publishes its partial sum of y^2 as ONE 64-bit word
// (call tag << 32 | fp32 bits), at its own place in the row's words; every
// wave of the row then polls all of the row's words, one lane per word,
// until all carry this call's tag, and adds them in a fixed tree order (the
// same in every wave: deterministic, no float atomics, and no barrier
// inside the workgroup). Because the tag travels in the same word as the
// value, no fence is needed, so no L2 writeback or invalidate is issued.
// The words stay in the XCD's L2 (workgroup-scope stores, non-temporal
// polls that the L1 does not keep) where the device deals workgroup ids to
// its XCDs round-robin, else they are device-scope. The tag is the row's
// epoch + 1, read at the start; the row's first wave advances the epoch once
// it has seen every word, which is after every workgroup of the row has
// read it. Epochs live in device memory, so graph replays stay correct.
//
// Co-residency. Polling requires all workgroups of a row to be resident at
// once. The host sizes the grid to at most half of the device's
// resident-workgroup capacity (the other half stays free for other streams'
// kernels) and, for larger row counts, walks the rows in rounds: in round k,
// workgroup w handles one (row, chunk) of a block of rows that the grid covers
// entirely, so every row's chunks are live together. The wait is bounded
// (spin_limit polls with s_sleep); a timeout is counted in the handle's error
// word and the wave goes on.
//
// XCD placement. Consecutive workgroup ids are dealt round-robin to the 8
// XCDs, so a row's chunks get ids congruent to the row mod 8: all
// workgroups of one row share one XCD's L2, where their polling stays.
#include <type_traits>

#include "coeff_epilogue.h"
#include "device_common.h"
#include "kernels.h"

namespace mhc {

constexpr int kHC = 4;
constexpr int kXcds = 8;
constexpr int kResidualOnlyBlock = 512;  // threads, at two elements per lane

struct BoundaryParams {
  // sublayer output: TP partials ...
  const uint4* xp;          // [tp][rows][hv]
  int tp;
  int scale_kt;             // MXFP8 scale layout (mx_scale_offset): 0 row-major, else 128x4 tiles
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
  int rows, hv, hidden, chunks;
  int xcd_handoff;          // the row's handoff words through its XCD's L2 (publish_word)
  uint4* layer_out;         // [rows][hv]
  uint2* mx_data;           // [rows][hv] (8 E4M3 codes per vector)
  uint8_t* mx_scale;        // [rows][hidden / 32] or swizzled (scale_kt)
  // row-RMS handoff
  unsigned long long* slots;  // [max_rows][slot_stride]
  unsigned* epoch;            // [max_rows][kEpochStride]
  unsigned* errors;           // [1]
  int slot_stride;
  int rows_per_round;         // rows per XCD per round
  int rounds;
  int spin_limit;
};
// The argument block of the undeferred kernels stays within 256 bytes (a step in launch
// cost was measured above it).
static_assert(sizeof(BoundaryParams) == 192, "BoundaryParams grew");

// Deferred coefficients: post, comb and pre come from a pending coefficient call's
// split-K partials, finished in the kernel; each row's first workgroup writes them out.
// A kernel argument of the deferred variants only (the others take an empty one, so
// that their argument block stays small).
struct DeferParams {
  CoeffEpilogue coef;
  float* def_pre;
  float* def_post;
  float* def_comb;
};
struct NoDefer {};
constexpr int kBoundaryPrefetch = 8;  // float4 of a row's partials fetched ahead per lane
template <bool DEFER>
using DeferArg = typename std::conditional<DEFER, DeferParams, NoDefer>::type;

// Deferred coefficients, wave 0 of the workgroup: finish row r's coefficient epilogue
// from the prefetched partials into s_coef (pre | post | comb, as coeff_row's slots); the
// row's first workgroup also writes them to the pending call's outputs. The workgroup
// reads s_coef after the next barrier.
__device__ __forceinline__ void deferred_finish(const DeferParams& d, int r, int c,
                                                const CoeffPrefetch<kBoundaryPrefetch>& f,
                                                float sc_l,
                                                float base_l, float* s_coef) {
  const int L = threadIdx.x;
  int slot;
  const float v = coeff_row_finish<true>(d.coef, r, L, f, sc_l, base_l, &slot);
  if (slot >= 0) {
    s_coef[slot] = v;
    if (c == 0) {
      if (slot < kHC) d.def_pre[r * kHC + slot] = v;
      else if (slot < 2 * kHC) d.def_post[r * kHC + slot - kHC] = v;
      else d.def_comb[r * kHC * kHC + slot - 2 * kHC] = v;
    }
  }
}

// One lane per vector of EL consecutive elements (EL = 8, 4 or 2: 16-, 8- or 4-byte
// vectors): the lane owns those elements of the row and all four streams of them (BS
// vectors per workgroup). Every kernel computes the new streams here; with HAS_PRE also
// the collapse, the row handoff and the layer input.
template <int BS, bool FINALIZE, bool HAS_PRE, bool MXFP8, int MODE, bool DEFER, int EL>
__device__ __forceinline__ void boundary_item_lane(const BoundaryParams& p_arg,
                                                   const float* __restrict__ post,
                                                   const float* __restrict__ comb,
                                                   const float* __restrict__ pre,
                                                   const int* __restrict__ idx,
                                                   const float* __restrict__ ew,
                                                   const DeferArg<DEFER>& dp, int r, int c,
                                                   float* s_coef, float sc_l, float base_l) {
  // with MXFP8 output, the sizes pass through an empty asm, so that what derives from them
  // is computed per row rather than hoisted out of the round loop and spilled (measured:
  // the headline call 4.35 -> 4.28 us; the kernels without MXFP8 measured level or slower)
  BoundaryParams p = p_arg;
  if constexpr (MXFP8)
    asm volatile("" : "+s"(p.tp), "+s"(p.top_k), "+s"(p.rows), "+s"(p.hv), "+s"(p.chunks));
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  static_assert(EL == 8 || EL == 4 || EL == 2, "a lane holds 8, 4 or 2 elements");
  using Vec = typename std::conditional<
      EL == 8, uint4, typename std::conditional<EL == 4, uint2, uint32_t>::type>::type;
  const int nv = p.hv * (8 / EL);  // vectors per row
  const Vec* xp = reinterpret_cast<const Vec*>(p.xp);
  const Vec* gp = reinterpret_cast<const Vec*>(p.g);
  const Vec* shp = reinterpret_cast<const Vec*>(p.shared);
  const Vec* res_in = reinterpret_cast<const Vec*>(p.res_in);
  Vec* res_out = reinterpret_cast<Vec*>(p.res_out);
  const Vec* norm_w = reinterpret_cast<const Vec*>(p.norm_w);
  Vec* layer_out = reinterpret_cast<Vec*>(p.layer_out);
  const int v = c * BS + tid;
  const bool active = v < nv;
  const int va = active ? v : 0;

  // the row's epoch and poison flag, read by every wave without a branch, first, so that
  // their latency hides under the data loads
  unsigned epoch_now = 0, poisoned = 0;
  if constexpr (HAS_PRE) {
    const unsigned long long ew = __hip_atomic_load(
        reinterpret_cast<const unsigned long long*>(p.epoch + (size_t)r * kEpochStride),
        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    epoch_now = (unsigned)ew;
    poisoned = (unsigned)(ew >> 32);
  }

  float x[EL];
#pragma unroll
  for (int e = 0; e < EL; ++e) x[e] = 0.f;
  int pk[8];
  float wk[8];
  if constexpr (FINALIZE) {
    // branch-free: slots past top_k re-read the row's last slot and are dropped at the
    // gathers. Only the loads here: the selects on them come after the streaming loads, so
    // that no wait for these scalar loads sits ahead of those
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int uu = u < p.top_k ? u : p.top_k - 1;
      pk[u] = idx[r * p.top_k + uu];
      wk[u] = ew[r * p.top_k + uu];
    }
  }
  float pst[kHC], cmb[kHC * kHC], pr[kHC];
  if constexpr (MODE == kBoundaryMix && !DEFER) {
#pragma unroll
    for (int i = 0; i < kHC; ++i) pst[i] = post[r * kHC + i];
#pragma unroll
    for (int i = 0; i < kHC * kHC; ++i) cmb[i] = comb[r * kHC * kHC + i];
  }
  if constexpr (HAS_PRE && MODE != kBoundaryFirst && !DEFER) {
#pragma unroll
    for (int i = 0; i < kHC; ++i) pr[i] = pre[r * kHC + i];
  }
  // the norm weight first: it is shared by every row, so it mostly hits in L2, and issued
  // ahead of the streaming loads it is back before them (measured: 0.2 us per call)
  Vec wv = {};
  if constexpr (HAS_PRE) wv = norm_w[va];
  Vec sv[kHC];
  if constexpr (MODE != kBoundaryFirst) {
#pragma unroll
    for (int j = 0; j < kHC; ++j) sv[j] = load_nt(res_in + ((size_t)r * kHC + j) * nv + va);
  }
  Vec xr = {};  // first: the embedding vector itself
  CoeffPrefetch<kBoundaryPrefetch> cf;
  if constexpr (DEFER)
    if (wave == 0) coeff_row_prefetch<true>(dp.coef, r, lane, cf);

  if constexpr (MODE == kBoundaryFirst) {
    xr = load_nt(xp + (size_t)r * nv + va);
    unpack_bf16(xr, x);
  } else if constexpr (MODE == kBoundaryHead) {
    // no sublayer output
  } else if constexpr (!FINALIZE) {
    // t ascending. In each full group of eight slices the loads issue back to back without
    // a branch, each address the previous one plus the slice stride; the stride passes
    // through an empty asm at every step, so that the compiler keeps one 64-bit add per
    // slice rather than forming each slice's offset as a 64-bit product in scalar
    // registers ahead of the first load (measured: ~90 scalar instructions before the
    // loads, the headline call 4.29 -> 4.06 us). A ragged last group takes the branchy form.
    const Vec* src = xp + (size_t)r * nv + va;
    const size_t slice = (size_t)p.rows * nv;
    size_t step = slice * sizeof(Vec);
    const int full = p.tp & ~7;
    for (int t0 = 0; t0 < full; t0 += 8) {
      Vec xv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        xv[u] = load_nt(src);
        asm volatile("" : "+s"(step));
        src = reinterpret_cast<const Vec*>(reinterpret_cast<const char*>(src) + step);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        float f[EL];
        unpack_bf16(xv[u], f);
#pragma unroll
        for (int e = 0; e < EL; ++e) x[e] += f[e];
      }
    }
    if (full < p.tp) {
      Vec xv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (full + u < p.tp) xv[u] = load_nt(src + (size_t)u * slice);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (full + u < p.tp) {
          float f[EL];
          unpack_bf16(xv[u], f);
#pragma unroll
          for (int e = 0; e < EL; ++e) x[e] += f[e];
        }
      }
    }
  } else {
    // k ascending, then the shared row
    const Vec shv = load_nt(shp + (size_t)r * nv + va);
    // every gather issued (a slot past top_k or out of range reads row 0 with weight 0, and
    // only slots below top_k are added); behind a branch each, the gathers had waited for
    // the slots one by one (measured: finalize + MXFP8 at 64 rows 5.93 -> 5.79 us). No
    // instruction crosses this point, so the slots' selects and the gather addresses,
    // which wait for the slots, stay behind the loads above
    __builtin_amdgcn_sched_barrier(0);
    Vec gv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool ok = u < p.top_k && pk[u] >= 0 && pk[u] < p.num_permuted;
      gv[u] = load_nt(gp + (size_t)(ok ? pk[u] : 0) * nv + va);
      if (!ok) wk[u] = 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (u < p.top_k) {
        float f[EL];
        unpack_bf16(gv[u], f);
#pragma unroll
        for (int e = 0; e < EL; ++e) x[e] = __builtin_fmaf(wk[u], f[e], x[e]);
      }
    }
    for (int k = 8; k < p.top_k; ++k) {  // slots beyond 8, in order
      const int pi = idx[r * p.top_k + k];
      const bool ok = pi >= 0 && pi < p.num_permuted;
      const float w = ok ? ew[r * p.top_k + k] : 0.f;
      const Vec g = load_nt(gp + (size_t)(ok ? pi : 0) * nv + va);
      float f[EL];
      unpack_bf16(g, f);
#pragma unroll
      for (int e = 0; e < EL; ++e) x[e] = __builtin_fmaf(w, f[e], x[e]);
    }
    float f[EL];
    unpack_bf16(shv, f);
#pragma unroll
    for (int e = 0; e < EL; ++e) x[e] += f[e];
  }
  if constexpr (MODE == kBoundaryMix) round_bf16(x);  // the reduced output is a bf16 tensor
  if constexpr (DEFER) {
    if (wave == 0) deferred_finish(dp, r, c, cf, sc_l, base_l, s_coef);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kHC; ++i) {
      pr[i] = s_coef[i];
      pst[i] = s_coef[kHC + i];
    }
#pragma unroll
    for (int i = 0; i < kHC * kHC; ++i) cmb[i] = s_coef[2 * kHC + i];
  }

  float sn[kHC][EL];
  if constexpr (MODE == kBoundaryFirst) {
    // every stream is the embedding, bit for bit
    Vec* out = res_out + (size_t)r * kHC * nv + v;
#pragma unroll
    for (int i = 0; i < kHC; ++i)
      if (active) store_nt(out + (size_t)i * nv, xr);
  } else if constexpr (MODE == kBoundaryHead) {
#pragma unroll
    for (int j = 0; j < kHC; ++j) unpack_bf16(sv[j], sn[j]);
  } else {
    Vec* out = res_out + (size_t)r * kHC * nv + v;
    float s[kHC][EL];
#pragma unroll
    for (int j = 0; j < kHC; ++j) unpack_bf16(sv[j], s[j]);
#pragma unroll
    for (int i = 0; i < kHC; ++i) {
#pragma unroll
      for (int e = 0; e < EL; ++e) {
        float a = pst[i] * x[e];
#pragma unroll
        for (int j = 0; j < kHC; ++j) a = __builtin_fmaf(cmb[i * kHC + j], s[j][e], a);
        sn[i][e] = a;
      }
      const Vec o = pack_bf16(sn[i]);
      if (active) store_nt(out + (size_t)i * nv, o);  // the streams do not wait for the RMS
      if constexpr (HAS_PRE) unpack_bf16(o, sn[i]);
    }
  }
  if constexpr (!HAS_PRE) return;

  float y[EL];
  float sq = 0.f;
  if constexpr (MODE == kBoundaryFirst) {
#pragma unroll
    for (int e = 0; e < EL; ++e) y[e] = x[e];  // the identity pre-mix
  } else {
#pragma unroll
    for (int e = 0; e < EL; ++e) {
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < kHC; ++j) a = __builtin_fmaf(pr[j], sn[j][e], a);
      y[e] = a;
    }
    // the head's collapse is a bf16 tensor of its own before the norm
    if constexpr (MODE == kBoundaryHead) round_bf16(y);
  }
#pragma unroll
  for (int e = 0; e < EL; ++e) sq = __builtin_fmaf(y[e], y[e], sq);
  if (!active) sq = 0.f;
  sq = wave_sum(sq);
  // the row handoff: every wave publishes its partial sum of y^2 as one word of the row
  // (chunk-major: word c * waves + wave), then waits for all of the row's words itself, one
  // lane per word, and adds them in a fixed tree order, so every wave of the row gets the
  // same bits without a barrier
  constexpr int kWaves = BS / kWave;
  const unsigned want = epoch_now + 1u;
  const bool xcd = p.xcd_handoff != 0;
  unsigned long long* row_slots = p.slots + (size_t)r * p.slot_stride;
  if (lane == 0)
    publish_word(row_slots + c * kWaves + wave,
                 ((unsigned long long)want << 32) | __float_as_uint(sq), xcd);
  // a row whose wait gave up once (a late wave of that call may have left a word with a tag
  // a later call wants) trusts no word until mhc_reset: the wait is skipped and the layer
  // input poisoned
  bool failed = poisoned != 0;
  float part = 0.f;
  const int words = p.chunks * kWaves;
  for (int k = lane; k < words && !failed; k += kWave) {
    unsigned long long wd;
    int spins = 0;
    for (;;) {
      wd = poll_word(row_slots + k, xcd);
      if ((unsigned)(wd >> 32) == want) break;
      if (++spins > p.spin_limit) {
        __hip_atomic_fetch_add(p.errors, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        failed = true;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    part += __uint_as_float((unsigned)wd);
  }
  float tot = wave_sum(part);
  // a wait that gave up makes this wave's share of the layer input NaN (and its MXFP8
  // scales the E8M0 NaN byte), so that the failure shows in the data, and marks the row
  // (word 1 of its epoch line) for the calls after it
  if (__ballot(failed) != 0) {
    tot = __builtin_nanf("");
    if (lane == 0 && !poisoned)
      __hip_atomic_store(p.epoch + (size_t)r * kEpochStride + 1, 1u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
  // every word of the row is in, so every workgroup of the row has read the epoch: the
  // row's first wave advances it
  if (c == 0 && wave == 0 && lane == 0)
    __hip_atomic_store(p.epoch + (size_t)r * kEpochStride, want, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  if (!active) return;
  const float inv = fast_rsq(tot * fast_rcp((float)p.hidden) + p.eps);
  float w[EL], o[EL];
  unpack_bf16(wv, w);
#pragma unroll
  for (int e = 0; e < EL; ++e) o[e] = (y[e] * inv) * w[e];
  const Vec ob = pack_bf16(o);
  store_nt(layer_out + (size_t)r * nv + v, ob);
  if constexpr (MXFP8) {
    // 32-element block = the 32 / EL consecutive lanes holding vectors v & ~(32/EL - 1) ..
    // (a quad at EL = 8, two quads at EL = 4, a 16-lane DPP row at EL = 2)
    constexpr int kPerBlock = 32 / EL;
    float q[EL];
    unpack_bf16(ob, q);
    // the block's largest magnitude, as the unsigned maximum of the magnitudes' bit
    // patterns (non-negative floats order as their bits): each step is then one DPP max,
    // with no LDS swizzle (measured: headline 4.06 -> 4.02 us). The steps: the quad's
    // xors, the half-row mirror (lane i <-> 7 - i: the other quad of the eight), and at
    // two per lane the rotation of the 16-lane row by 8
    uint32_t amax = 0;
#pragma unroll
    for (int e = 0; e < EL; ++e) amax = max(amax, __float_as_uint(q[e]) & 0x7FFFFFFFu);
    amax = max(amax, dpp_u32<kDppQuadXor1>(amax));
    amax = max(amax, dpp_u32<kDppQuadXor2>(amax));
    if constexpr (EL <= 4) amax = max(amax, dpp_u32<kDppRowHalfMirror>(amax));
    if constexpr (EL == 2) amax = max(amax, dpp_u32<kDppRowRor8>(amax));
    const int ex = e8m0_exponent(amax);
    const float sc = __uint_as_float((uint32_t)(127 - ex) << 23);
    // |q| * 2^-e <= 448 by the choice of e: in range, exact scaling
    if constexpr (EL == 8) {
      const uint32_t lo = cvt_pk4_e4m3(q[0] * sc, q[1] * sc, q[2] * sc, q[3] * sc);
      const uint32_t hi = cvt_pk4_e4m3(q[4] * sc, q[5] * sc, q[6] * sc, q[7] * sc);
      store_nt(p.mx_data + (size_t)r * p.hv + v, make_uint2(lo, hi));
    } else if constexpr (EL == 4) {
      const uint32_t lo = cvt_pk4_e4m3(q[0] * sc, q[1] * sc, q[2] * sc, q[3] * sc);
      store_nt(reinterpret_cast<uint32_t*>(p.mx_data) + (size_t)r * nv + v, lo);
    } else {
      const uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[0] * sc, q[1] * sc, 0, false);
      store_nt(reinterpret_cast<uint16_t*>(p.mx_data) + (size_t)r * nv + v, (uint16_t)lo);
    }
    if ((v & (kPerBlock - 1)) == 0)
      p.mx_scale[mx_scale_offset(r, v / kPerBlock, p.hidden / 32, p.scale_kt)] =
          inv == inv ? (uint8_t)(ex + 127) : (uint8_t)0xFF;  // NaN: a wait gave up
  }
}

// The deferred variants are held to at least 4 waves per SIMD (at most 128 VGPRs), as
// the others are without a hint, so that a 128-row call keeps one round.
template <int BS, bool FINALIZE, bool HAS_PRE, bool MXFP8, int MODE, bool DEFER, int EL = 8>
__global__ __launch_bounds__(BS, DEFER ? 4 : 1) void boundary_kernel(const BoundaryParams p,
                                                      const float* __restrict__ post,
                                                      const float* __restrict__ comb,
                                                      const float* __restrict__ pre,
                                                      const int* __restrict__ idx,
                                                      const float* __restrict__ ew,
                                                      const DeferArg<DEFER> dp) {
  prefetch_kernargs<sizeof(BoundaryParams) + 5 * sizeof(void*) + sizeof(DeferArg<DEFER>)>();
  __shared__ float s_coef[2 * kHC + kHC * kHC];
  float sc_l = 0.f, base_l = 0.f;  // deferred coefficients: this lane's scale and base
  if constexpr (DEFER) coeff_lane_scale_base(dp.coef, threadIdx.x & (kWave - 1), &sc_l, &base_l);
  const int wg = blockIdx.x;
  const int xcd = wg % kXcds;
  const int local = wg / kXcds;
  const int c = local % p.chunks;
  const int jr = local / p.chunks;  // which row of this XCD's block in a round
  for (int round = 0; round < p.rounds; ++round) {
    const int r = (round * p.rows_per_round + jr) * kXcds + xcd;
    if (r >= p.rows) break;  // uniform per workgroup; later rounds only go higher
    // the lane kernels have no barrier after the deferred coefficients are read: one here
    // keeps a later round's finish from overwriting them while a wave still reads them
    // (the residual-only calls take one round, so it never runs for them)
    if (DEFER && round > 0) __syncthreads();
    boundary_item_lane<BS, FINALIZE, HAS_PRE, MXFP8, MODE, DEFER, EL>(
        p, post, comb, pre, idx, ew, dp, r, c, s_coef, sc_l, base_l);
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
  store_nt(out + i, pack8_round(acc));
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
template <int BS, bool FIN, bool PRE, bool MX, int MODE = kBoundaryMix, bool DEFER = false,
          int EL = 8>
static hipError_t launch_one(const BoundaryParams& p, const DeferParams& d, int grid,
                             hipStream_t st) {
  DeferArg<DEFER> dp;
  if constexpr (DEFER) dp = d;
  hipLaunchKernelGGL((boundary_kernel<BS, FIN, PRE, MX, MODE, DEFER, EL>), dim3(grid), dim3(BS), 0,
                     st, p, p.post, p.comb, p.pre, p.idx, p.ew, dp);
  return hipGetLastError();
}

template <int BS, bool DEFER>
static hipError_t launch_mix(const BoundaryParams& p, const DeferParams& d, bool fin, bool pre,
                             bool mx, int el, int grid, hipStream_t st) {
  if (!pre) {  // residual-only: always two elements per lane at 512 threads
    if constexpr (BS == kResidualOnlyBlock)
      if (el == 2)
        return fin ? launch_one<BS, true, false, false, kBoundaryMix, DEFER, 2>(p, d, grid, st)
                   : launch_one<BS, false, false, false, kBoundaryMix, DEFER, 2>(p, d, grid, st);
    return hipErrorInvalidValue;
  }
  if constexpr (BS == 512) {
    if (el == 2 && pre) {  // two elements per lane (the layer-input kernels)
      if (!fin)
        return mx ? launch_one<BS, false, true, true, kBoundaryMix, DEFER, 2>(p, d, grid, st)
                  : launch_one<BS, false, true, false, kBoundaryMix, DEFER, 2>(p, d, grid, st);
      return mx ? launch_one<BS, true, true, true, kBoundaryMix, DEFER, 2>(p, d, grid, st)
                : launch_one<BS, true, true, false, kBoundaryMix, DEFER, 2>(p, d, grid, st);
    }
  }
  if constexpr (BS >= 256) {
    if (el == 4 && pre) {  // four elements per lane (the layer-input kernels)
      if (!fin)
        return mx ? launch_one<BS, false, true, true, kBoundaryMix, DEFER, 4>(p, d, grid, st)
                  : launch_one<BS, false, true, false, kBoundaryMix, DEFER, 4>(p, d, grid, st);
      return mx ? launch_one<BS, true, true, true, kBoundaryMix, DEFER, 4>(p, d, grid, st)
                : launch_one<BS, true, true, false, kBoundaryMix, DEFER, 4>(p, d, grid, st);
    }
  }
  if (!fin)
    return mx ? launch_one<BS, false, true, true, kBoundaryMix, DEFER>(p, d, grid, st)
              : launch_one<BS, false, true, false, kBoundaryMix, DEFER>(p, d, grid, st);
  return mx ? launch_one<BS, true, true, true, kBoundaryMix, DEFER>(p, d, grid, st)
            : launch_one<BS, true, true, false, kBoundaryMix, DEFER>(p, d, grid, st);
}

template <int BS>
static hipError_t launch_bs(const BoundaryParams& p, const DeferParams& d, bool fin, bool pre,
                            bool mx, int mode, bool defer, int el, int grid, hipStream_t st) {
  if constexpr (BS == 512) {
    if (el == 2 && mode == kBoundaryHead)
      return mx ? launch_one<BS, false, true, true, kBoundaryHead, false, 2>(p, d, grid, st)
                : launch_one<BS, false, true, false, kBoundaryHead, false, 2>(p, d, grid, st);
  }
  if constexpr (BS >= 256) {
    if (el == 4 && mode == kBoundaryHead)
      return mx ? launch_one<BS, false, true, true, kBoundaryHead, false, 4>(p, d, grid, st)
                : launch_one<BS, false, true, false, kBoundaryHead, false, 4>(p, d, grid, st);
  }
  if (mode == kBoundaryFirst)
    return mx ? launch_one<BS, false, true, true, kBoundaryFirst>(p, d, grid, st)
              : launch_one<BS, false, true, false, kBoundaryFirst>(p, d, grid, st);
  if (mode == kBoundaryHead)
    return mx ? launch_one<BS, false, true, true, kBoundaryHead>(p, d, grid, st)
              : launch_one<BS, false, true, false, kBoundaryHead>(p, d, grid, st);
  return defer ? launch_mix<BS, true>(p, d, fin, pre, mx, el, grid, st)
               : launch_mix<BS, false>(p, d, fin, pre, mx, el, grid, st);
}

template <int BS, bool FIN, bool PRE, bool MX, int MODE = kBoundaryMix, bool DEFER = false,
          int EL = 8>
static int occupancy_one() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &n, boundary_kernel<BS, FIN, PRE, MX, MODE, DEFER, EL>, BS, 0) != hipSuccess)
    return 0;
  return n;
}

template <int BS>
static int occupancy_bs() {
  // the polling variants only; the smallest of them bounds the co-resident grid
  int n = occupancy_one<BS, false, true, false>();
  n = min(n, occupancy_one<BS, false, true, true>());
  n = min(n, occupancy_one<BS, true, true, false>());
  n = min(n, occupancy_one<BS, true, true, true>());
  n = min(n, occupancy_one<BS, false, true, false, kBoundaryMix, true>());
  n = min(n, occupancy_one<BS, false, true, true, kBoundaryMix, true>());
  n = min(n, occupancy_one<BS, true, true, false, kBoundaryMix, true>());
  n = min(n, occupancy_one<BS, true, true, true, kBoundaryMix, true>());
  n = min(n, occupancy_one<BS, false, true, true, kBoundaryFirst>());
  n = min(n, occupancy_one<BS, false, true, true, kBoundaryHead>());
  if constexpr (BS >= 256) {
    n = min(n, occupancy_one<BS, false, true, false, kBoundaryMix, false, 4>());
    n = min(n, occupancy_one<BS, false, true, true, kBoundaryMix, false, 4>());
    n = min(n, occupancy_one<BS, true, true, false, kBoundaryMix, false, 4>());
    n = min(n, occupancy_one<BS, true, true, true, kBoundaryMix, false, 4>());
    n = min(n, occupancy_one<BS, false, true, false, kBoundaryMix, true, 4>());
    n = min(n, occupancy_one<BS, false, true, true, kBoundaryMix, true, 4>());
    n = min(n, occupancy_one<BS, true, true, false, kBoundaryMix, true, 4>());
    n = min(n, occupancy_one<BS, true, true, true, kBoundaryMix, true, 4>());
    n = min(n, occupancy_one<BS, false, true, true, kBoundaryHead, false, 4>());
  }
  if constexpr (BS == 512) {
    n = min(n, occupancy_one<BS, false, true, false, kBoundaryMix, false, 2>());
    n = min(n, occupancy_one<BS, false, true, true, kBoundaryMix, false, 2>());
    n = min(n, occupancy_one<BS, true, true, false, kBoundaryMix, false, 2>());
    n = min(n, occupancy_one<BS, true, true, true, kBoundaryMix, false, 2>());
    n = min(n, occupancy_one<BS, false, true, false, kBoundaryMix, true, 2>());
    n = min(n, occupancy_one<BS, false, true, true, kBoundaryMix, true, 2>());
    n = min(n, occupancy_one<BS, true, true, false, kBoundaryMix, true, 2>());
    n = min(n, occupancy_one<BS, true, true, true, kBoundaryMix, true, 2>());
    n = min(n, occupancy_one<BS, false, true, true, kBoundaryHead, false, 2>());
  }
  return n;
}

int boundary_resident_wgs_per_cu(int block) {
  switch (block) {
    case 128: return occupancy_bs<128>();
    case 256: return occupancy_bs<256>();
    case 512: return occupancy_bs<512>();
    default: return 0;
  }
}

int boundary_chunks(int hidden, int block) {
  const int hv = hidden / 8;  // 16-byte vectors; `block` of them per workgroup
  return (hv + block - 1) / block;
}

int boundary_handoff_words(int hidden) {
  return (boundary_chunks(hidden, 128) * (512 / kWave) + 15) / 16 * 16;
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
  const bool pre = L.pre != nullptr || L.mode == kBoundaryFirst;  // a layer input is written
  const int row_blocks = (L.rows + kXcds - 1) / kXcds;  // rows per XCD in total
  // rows per XCD per round: a round may use at most half of the XCD's resident workgroups
  // (at least one row: a row's chunks fit half an XCD, checked at handle creation)
  auto rows_per_round = [&](int max_wgs, int chunks) {
    int rpr = (max_wgs / 2) / chunks;
    if (rpr < 1) rpr = 1;
    return rpr > row_blocks ? row_blocks : rpr;
  };
  // fewer elements per lane where asked for (the kernels that write a layer input, at
  // block_n = block * 8 / lane_elems threads: the same chunks as `block` at eight), unless
  // the larger workgroups would take more rounds (measured: a second round costs more than
  // the shorter per-lane work saves). Deferred and undeferred calls choose alike, so their
  // results stay bit-identical. Not the first layer's entry, which has almost no arithmetic
  // to share (measured 4.19 at eight against 4.22 us at four per lane, 32 rows).
  // (the residual-only kernels: 512 threads at two per lane, the chunks of 128 at eight)
  const int chunks8 = boundary_chunks(L.hidden, pre ? L.block : kResidualOnlyBlock / 4);
  bool narrow = L.lane_elems < 8 && pre && L.mode != kBoundaryFirst && L.block_n >= 256;
  if (narrow) {
    const int r8 = rows_per_round(L.max_wgs_per_xcd, chunks8);
    const int rn = rows_per_round(L.max_wgs_per_xcd_n, chunks8);
    narrow = (row_blocks + rn - 1) / rn <= (row_blocks + r8 - 1) / r8;
  }
  const int el = !pre ? 2 : (narrow ? L.lane_elems : 8);
  const int block = !pre ? kResidualOnlyBlock : (narrow ? L.block_n : L.block);
  const int max_wgs_per_xcd = narrow ? L.max_wgs_per_xcd_n : L.max_wgs_per_xcd;
  p.chunks = chunks8;
  p.layer_out = reinterpret_cast<uint4*>(L.layer_input_out);
  p.mx_data = reinterpret_cast<uint2*>(L.mx_data_out);
  p.mx_scale = L.mx_scale_out;
  p.scale_kt = L.scale_kt;
  p.slots = L.slots;
  p.epoch = L.epoch;
  p.errors = L.errors;
  p.slot_stride = L.slot_stride;
  p.spin_limit = L.spin_limit;
  p.xcd_handoff = L.xcd_handoff ? 1 : 0;
  DeferParams d;
  d.coef = L.coef;
  d.def_pre = L.defer ? L.pre_pending : nullptr;
  d.def_post = L.defer ? const_cast<float*>(L.post) : nullptr;
  d.def_comb = L.defer ? const_cast<float*>(L.comb) : nullptr;
  const bool fin = L.gemm2_permuted != nullptr;
  const bool mx = L.mx_data_out != nullptr;
  if (pre) {
    const int rpr = rows_per_round(max_wgs_per_xcd, p.chunks);
    p.rows_per_round = rpr;
    p.rounds = (row_blocks + rpr - 1) / rpr;
  } else {
    p.rows_per_round = row_blocks;
    p.rounds = 1;
  }
  // every wave of a row owns one handoff word of the row's slot line(s)
  if (pre && p.chunks * (block / kWave) > p.slot_stride) return hipErrorInvalidValue;
  const int grid = kXcds * p.rows_per_round * p.chunks;
  switch (block) {
    case 128: return launch_bs<128>(p, d, fin, pre, mx, L.mode, L.defer, el, grid, stream);
    case 256: return launch_bs<256>(p, d, fin, pre, mx, L.mode, L.defer, el, grid, stream);
    case 512: return launch_bs<512>(p, d, fin, pre, mx, L.mode, L.defer, el, grid, stream);
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

namespace {
__global__ __launch_bounds__(64) void xcd_probe_kernel(unsigned* out) {
  unsigned x;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
  if (threadIdx.x == 0) out[blockIdx.x] = x & 0xFu;
}
}  // namespace

hipError_t probe_xcd_round_robin(unsigned* buf, bool* round_robin) {
  *round_robin = false;
  hipLaunchKernelGGL(xcd_probe_kernel, dim3(kXcdProbeWgs), dim3(64), 0, nullptr, buf);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  unsigned h[kXcdProbeWgs];
  e = hipMemcpy(h, buf, sizeof(h), hipMemcpyDeviceToHost);  // synchronizes
  if (e != hipSuccess) return e;
  bool ok = true;
  for (int i = 0; i < kXcdProbeWgs; ++i) ok = ok && h[i] == h[i % kXcds];
  for (int i = 0; i < kXcds; ++i)
    for (int j = 0; j < i; ++j) ok = ok && h[i] != h[j];  // eight distinct XCDs
  *round_robin = ok;
  return hipSuccess;
}

}  // namespace mhc
