// The boundary fused with the next sublayer's coefficient call, for gfx950: one kernel
// computes what mhc_boundary (or mhc_finalize) and then mhc_pre_coeffs on its new streams
// compute, without the coefficient call's re-read of the streams or its launches.
//
// Pages: boundary page, Boundaries.sublayer (the boundary is followed by the next
// sublayer's coefficient call on the streams it returns) and Boundaries._pre (that
// call's arguments); the arithmetic of each step is stated in include/mhc.h.
//
// Work decomposition. A workgroup of 512 threads (8 waves) owns a tile of 16 rows by
// 256 hidden elements (one chunk). For every global load and store, the 32 lanes of a half
// wave own one row's 32 vectors of the chunk (512 contiguous bytes), with all four streams
// of them: the same per-lane dataflow as the boundary's layer-input kernels (partial
// slices or gathered expert rows, mHC post, collapse, RMSNorm, MXFP8), in the same
// arithmetic order, so the new streams are bit-identical to mhc_boundary's. (A layout
// with 16 rows across consecutive lanes, the MFMA operand layout, made every 16-lane
// memory pass touch 16 cache lines: 25.8 us per 128-row call against 17.8 with this one,
// before the later changes.)
//
// The projection. The bf16 new streams are also written to LDS ([stream][row][vector],
// rows padded against bank conflicts). Wave w then reads, for each stream i, 16 rows by
// elements 32w .. 32w + 31 of the chunk as the B operand of one v_mfma_f32_16x16x32_bf16
// (lane = row + 16 x 8-element group; N = rows, K = 32 elements); the A operand is fn^T
// over the same elements, staged in LDS (the chunk's fn rows, 4 x 256 x 24 bf16, copied
// with 16-byte loads and transposed to [logit][k]). Eight MFMAs per wave (4 streams x
// logits 0..15 and 16..31) give the wave's partial logits of the 16 rows; the eight
// waves' partials are added in wave order. Only the bf16 values the call stores enter the
// projection, as in mhc_pre_coeffs on the stored streams.
//
// The handoff. Every workgroup publishes, per row of its tile, the partial sum of y^2 (for
// the layer input's RMS; first, one contiguous line per workgroup), then the 24 partial
// logits and the partial sum of the new streams' squares (for the coefficients' RMS),
// each as a 64-bit word (call tag << 32 | fp32 bits, relaxed device-scope store). Each
// half wave then reads its row's y^2 words, one chunk per lane (so chunks <= 32), until
// all carry the call's tag, adds them in a fixed tree order (deterministic) and writes
// its share of the layer input: no barrier. Workgroup c of the tile also finishes the
// coefficients of rows c, c + chunks, ...: lanes 0..24 of one wave read the row's 25
// coefficient words of every chunk, add them in chunk order and run the coefficient
// epilogue (coeff_epilogue.h), writing the next pre, post and comb; it does so before its
// own layer-input stores, since a wait for loads also waits for the stores before them.
// Tags are the rows' epochs + 1 (the same epochs as the boundary's handoff); chunk 0
// advances a row's epoch once it has seen the row's every word, i.e. after every
// workgroup of the tile has read it. A word's place depends only on its row and chunk
// (the layout is sized for the handle's rows), so a stale word carries an older tag.
//
// Co-residency and placement as the boundary's: a tile's chunks get workgroup ids
// congruent mod 8 (one XCD, one L2), the grid holds at most the device's resident
// capacity of this kernel, rows beyond it are walked in rounds, and every wait is bounded.
#include "coeff_epilogue.h"
#include "device_common.h"
#include "kernels.h"

namespace mhc {

namespace {

constexpr int kN = 4;
constexpr int kXcd = 8;
constexpr int kTileRows = 16;
constexpr int kTileWaves = 8;
constexpr int kTileThreads = kTileWaves * kWave;          // 512
constexpr int kTileVecs = kTileThreads / kTileRows;       // 32 vectors of a row per chunk
constexpr int kTileH = kTileVecs * 8;                     // 256 elements per chunk
constexpr int kWordsPerRow = 2 + kCoefNC;                 // y^2, 24 logits, v^2
constexpr int kFnK = kN * kTileH;                         // 1024 k values per chunk
constexpr int kFnLd = kFnK + 8;                           // padded LDS row of fn^T
constexpr int kFnVecs = kFnK * kCoefNC / 8 / kTileThreads;  // 6 16-byte vectors per thread
constexpr int kFinishBatch = 32;                          // chunks per row at most (a half wave)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct TileParams {
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
  const float4* post;       // [rows] (4 floats)
  const float4* comb;       // [rows][4] (16 floats)
  const float4* pre;        // [rows] (4 floats)
  const uint4* norm_w;      // [hv]
  float eps;
  int rows, hv, chunks;     // hidden = 8 hv
  uint4* layer_out;         // [rows][hv]
  uint2* mx_data;           // [rows][hv]
  uint8_t* mx_scale;        // [rows][hidden / 32] or swizzled (scale_kt)
  // the next coefficients
  const uint4* fn;          // [4 * hidden][24] bf16, 3 vectors per k row
  const float* scale;       // [3]
  const float* base;        // [24]
  float rms_eps, pre_eps, sk_eps, alpha;
  int iters;
  int groups;               // 0: a tile's chunks on one XCD; else chunk c on XCD c % 8, with
                            // `groups` = ceil(chunks / 8) chunks of each tile per XCD
  union {
    float* next_pre;        // [rows][4]
    float* part_out;        // DEFER_OUT: partials of the next call (coeff_part_index, part_ks)
  };
  float* next_post;         // [rows][4]
  float* next_comb;         // [rows][16]
  // handoff
  unsigned long long* words;  // y^2 words [tiles][chunks][16], then coefficient words
                              // [tiles][chunks][16][25]
  unsigned* epoch;            // [max_rows][kEpochStride]
  unsigned* errors;
  int tile_cap, tiles_per_round, rounds, spin_limit;  // tile_cap: tiles of the scratch
};
// The whole argument block of the undeferred kernels: at most 256 bytes (a step in launch
// cost was measured above it).
static_assert(sizeof(TileParams) == 256, "TileParams grew");

// Handoff words, tile-major: per (tile, chunk) the 16 rows' sums of y^2, then per (tile,
// chunk, row) the 25 coefficient partials (24 logits, the sum of v^2). One workgroup's
// words are contiguous.
// (The words of a handle of at most 1024 rows and 32 chunks per row: a 32-bit index.)
__device__ __forceinline__ uint32_t ysq_index(const TileParams& p, int tile, int c, int rr) {
  return ((uint32_t)tile * p.chunks + c) * kTileRows + rr;
}
__device__ __forceinline__ uint32_t coef_index(const TileParams& p, int tile, int c, int rr,
                                               int v) {
  // after the y^2 words of every tile the handle holds: each word's place belongs to one
  // row whatever the call's row count, so a stale word carries an older tag of that row
  const uint32_t base = (uint32_t)p.tile_cap * p.chunks * kTileRows;
  return base + (((uint32_t)tile * p.chunks + c) * kTileRows + rr) * kCoefPartW + v;
}
__device__ __forceinline__ unsigned long long* word_at(const TileParams& p, uint32_t i) {
  return byte_at(p.words, i * 8u);
}

__device__ __forceinline__ unsigned long long tagged(unsigned tag, float f) {
  return ((unsigned long long)tag << 32) | __float_as_uint(f);
}

// Sum over the 32 lanes of each half wave (a tile row's lanes), in a fixed order.
__device__ __forceinline__ float half_wave_sum(float v) {
  v += dpp_f32<kDppQuadXor1>(v);
  v += dpp_f32<kDppQuadXor2>(v);
  v += dpp_f32<kDppRowRor4>(v);
  v += dpp_f32<kDppRowRor8>(v);
  return v + __shfl_xor(v, 16, kWave);
}

// A pending coefficient call finished in this kernel: its epilogue arguments, with `part`
// its per-chunk partial sums (coeff_part_index, ks_count <= 32) written by the previous
// fused kernel. A kernel argument of those variants only.
struct TileDeferIn {
  CoeffEpilogue coef;
};

// The coefficient epilogue of two rows in one wave: half h (lanes 32h .. 32h + 31) holds
// row h's sums (lane 32h + l: value l, as coeff_from_sums's lane l), and row h's comb sits
// in the upper DPP row of its half (lanes 32h + 16 .. 32h + 31), so the Sinkhorn steps
// of both rows run in the same instructions. Per value, the operations and their order
// are coeff_from_sums's, so the results are bit-identical. Returns this lane's value and
// sets *slot (0..3 pre, 4..7 post, 8..23 comb of the half's row, -1 none).
__device__ __forceinline__ float coeff_two_rows(const CoeffEpilogue& e, int L, float acc,
                                                float sc_l, float base_l, int* slot) {
  const int l = L & 31, hb = L & 32;
  const float ss = __shfl(acc, hb + kCoefNC, kWave);
  const float inv = fast_rsq(ss * fast_rcp((float)e.K) + e.rms_eps);
  float lp = 0.f;
  if (l < kCoefNC) lp = (acc * inv) * sc_l + base_l;
  float out = 0.f;
  *slot = -1;
  if (l < kCoefN) {
    out = fast_rcp(1.0f + fast_exp(-lp)) + e.pre_eps;
    *slot = l;
  } else if (l < 2 * kCoefN) {
    out = e.alpha * fast_rcp(1.0f + fast_exp(-lp));
    *slot = l;
  }
  const int ce = l - 16;  // comb entry (i, j) = 4i + j at lane 32h + 16 + 4i + j
  float a = __shfl(lp, hb + 2 * kCoefN + (ce & 15), kWave);
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
  if (ce >= 0) {
    out = a;
    *slot = 2 * kCoefN + ce;
  }
  return out;
}

struct TileShared {
  uint16_t fnT[kCoefNC][kFnLd];                 // fn^T of the chunk, [logit][k]
  uint4 sT[kN][kTileRows][kTileVecs + 1];       // new streams, bf16, padded rows
  float red[kTileWaves][kTileRows][kCoefNC];    // per-wave partial logits
  float rowsum[kTileRows][2];                   // per-row sum of y^2, of v^2
  unsigned want[kTileRows];
  unsigned poisoned[kTileRows];  // the rows' poison flags (a wait of the row gave up)
  float4 cf[kTileRows][kCoefNC / 4];            // a pending call's coefficients (pre|post|comb)
};

// DEFER: 0 the next coefficients finished in the kernel; 1 left as partial sums (DEFER_OUT);
// 2 also this call's post, comb and pre finished here from the pending call's partial sums
// (DEFER_IN) instead of read.
template <bool FINALIZE, bool MXFP8, int DEFER>
__device__ __forceinline__ void tile_item(const TileParams& p_arg, const CoeffEpilogue& coef,
                                          const TileDeferIn* din_arg, int tile, int c,
                                          TileShared& S, float sc_l, float base_l, float dsc_l,
                                          float dbase_l) {
  // the sizes that the per-slot offsets and bounds derive from pass through an empty asm
  // too, for the same reason as the indices below: hoisted, those uniform values were
  // spilled into vector lanes (112 lane moves in the deferred TP kernel, 4 now)
  TileParams p = p_arg;
  asm volatile("" : "+s"(p.tp), "+s"(p.top_k), "+s"(p.rows), "+s"(p.hv), "+s"(p.chunks));
  TileDeferIn dcopy;
  const TileDeferIn* din = din_arg;
  if constexpr (DEFER == 2) {
    dcopy = *din_arg;
    asm volatile("" : "+s"(dcopy.coef.ks_count));
    din = &dcopy;
  }
  constexpr bool DEFER_OUT = DEFER >= 1;
  constexpr bool DEFER_IN = DEFER == 2;
  // the thread and chunk indices pass through an empty asm, so what derives from them is
  // computed here, per item: hoisted before the round loop (which mostly runs once) it
  // held scalar registers across the kernel, spilled them into vector lanes and kept
  // ~600 instructions ahead of the first loads
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  asm volatile("" : "+s"(c));
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  // global traffic: the 32 lanes of a half wave own one row's 32 vectors of the chunk
  const int m = tid >> 5;           // row of the tile
  const int vl = tid & 31;          // vector of the chunk
  const int row0 = tile * kTileRows;
  const int r = row0 + m;
  const int v = c * kTileVecs + vl;
  const bool row_ok = r < p.rows;
  const bool active = row_ok && v < p.hv;
  const int rl = row_ok ? r : 0;    // loads of inactive lanes stay in bounds
  const int va = v < p.hv ? v : 0;

  // Every load below is unconditional, with indices clamped into bounds (results of
  // out-of-range lanes are dropped later): a load behind a lane-dependent branch makes the
  // compiler wait for it before going on, which serializes the loads.
  // the rows' epochs (the call tag), kept in a register until the loads are issued
  // with the row's poison flag (word 1 of its epoch line): set once a wait of the row gave
  // up, after which no handoff word of the row is trusted until mhc_reset (a late workgroup
  // of that call may have left a word with a tag a later call wants)
  const unsigned long long ew = __hip_atomic_load(
      reinterpret_cast<const unsigned long long*>(
          p.epoch + (size_t)min(row0 + (tid & 15), p.rows - 1) * kEpochStride),
      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const unsigned epoch_now = (unsigned)ew;
  // the finalize's expert slots next: the gathers wait for them, and a wait covers every
  // load issued before (slots past top_k re-read the row's last one and get weight 0)
  int pk[8];
  float wk[8];
  if constexpr (FINALIZE) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int uu = u < p.top_k ? u : p.top_k - 1;
      const uint32_t o = ((uint32_t)rl * p.top_k + uu) * 4u;
      const int pi = *byte_at(p.idx, o);
      const float w = *byte_at(p.ew, o);
      pk[u] = u < p.top_k ? pi : -1;
      wk[u] = u < p.top_k ? w : 0.f;
    }
  }

  // --- DEFER_IN: the pending call's partial sums of this lane's row (the half wave's), value
  // vl (lanes past 24 repeat value 24), first: their wait then leaves the loads below in flight
  float4 dpart[kFinishBatch / 4];
  if constexpr (DEFER_IN) {
    const CoeffEpilogue& e = din->coef;
    const int Lc = min(vl, kCoefPartW - 1);
    const int last = e.ks_count / 4 - 1;  // past it: in-bounds repeats, never added
#pragma unroll
    for (int u = 0; u < kFinishBatch / 4; ++u) dpart[u] = coeff_quad(e, rl, Lc, u < last ? u : last);
  }

  // --- loads: fn slice (mostly L2 hits), the row's mixes, norm weight, streams, sublayer
  uint4 fv[kFnVecs];
#pragma unroll
  for (int j = 0; j < kFnVecs; ++j) {
    const int q = tid + j * kTileThreads;        // < 4 * 256 * 3
    const int i = q / (kTileH * 3), rem = q % (kTileH * 3);
    const int kk = rem / 3, part = rem % 3;
    const int h = min(c * kTileH + kk, (p.hv * 8) - 1);  // past the end: zeroed below
    fv[j] = *byte_at(p.fn, (((uint32_t)i * (p.hv * 8) + h) * 3 + part) * 16u);
  }
  float4 pst4, cmb4[kN], pr4;
  if constexpr (!DEFER_IN) {
    pst4 = *byte_at(p.post, (uint32_t)rl * 16u);
#pragma unroll
    for (int i = 0; i < kN; ++i) cmb4[i] = *byte_at(p.comb, ((uint32_t)rl * kN + i) * 16u);
    pr4 = *byte_at(p.pre, (uint32_t)rl * 16u);
  }
  // DEFER_IN: the pending call's coefficients of rows 2 wave and 2 wave + 1 (this wave's
  // halves), from their partial sums added in chunk order; into LDS, from which each half
  // reads its row's (wave-local: no barrier). Run while this item's loads are in flight.
  // Chunk 0 writes them to the pending call's outputs at the end of the item (a store
  // here would hold up every later wait for loads).
  auto finish_pending = [&]() {
    const CoeffEpilogue& e = din->coef;
    const int n4 = e.ks_count / 4;
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < kFinishBatch / 4; ++u)
      if (u < n4) acc = (((acc + dpart[u].x) + dpart[u].y) + dpart[u].z) + dpart[u].w;
    int slot;
    const float val = coeff_two_rows(e, lane, acc, dsc_l, dbase_l, &slot);
    float* cf = reinterpret_cast<float*>(&S.cf[m][0]);
    if (slot >= 0) cf[slot] = val;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    pr4 = S.cf[m][0];
    pst4 = S.cf[m][1];
#pragma unroll
    for (int i = 0; i < kN; ++i) cmb4[i] = S.cf[m][2 + i];
  };
  // per-lane byte offsets in 32 bits (the tile kernel's tensors are below 4 GiB: rows <= 1024,
  // hidden <= 8192, tp <= 64, num_permuted * hidden * 2 < 2^32, checked by the host)
  const uint32_t row_off = ((uint32_t)rl * p.hv + va) * 16u;  // [rows][hv] tensors
  const uint4 wv = *byte_at(p.norm_w, (uint32_t)va * 16u);
  uint4 sv[kN];
#pragma unroll
  for (int j = 0; j < kN; ++j)
    sv[j] = load_nt(byte_at(p.res_in, (((uint32_t)rl * kN + j) * p.hv + va) * 16u));

  // fn slice -> LDS, transposed to [logit][k] (k = stream * 256 + element of the chunk); run
  // once every load of the item is issued, while the sublayer output is still in flight (the
  // fn vectors were loaded first), so that this work is off the arithmetic that follows
  // the loads, where every wave of the CU competes for the vector units
  auto stage_fn = [&]() {
#pragma unroll
    for (int j = 0; j < kFnVecs; ++j) {
      const int q = tid + j * kTileThreads;
      const int i = q / (kTileH * 3), rem = q % (kTileH * 3);
      const int kk = rem / 3, c0 = (rem % 3) * 8;
      const bool ok = c * kTileH + kk < (p.hv * 8);
      const uint32_t u[4] = {ok ? fv[j].x : 0u, ok ? fv[j].y : 0u, ok ? fv[j].z : 0u,
                             ok ? fv[j].w : 0u};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        S.fnT[c0 + 2 * e][i * kTileH + kk] = (uint16_t)(u[e] & 0xFFFFu);
        S.fnT[c0 + 2 * e + 1][i * kTileH + kk] = (uint16_t)(u[e] >> 16);
      }
    }
  };
  float x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = 0.f;
  if constexpr (!FINALIZE) {
    // t ascending
    const uint32_t slice = (uint32_t)p.rows * p.hv * 16u;
    auto add_batch = [&](int t0, const uint4* xv) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (t0 + u < p.tp) {
          float f[8];
          unpack8(xv[u], f);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] += f[e];
        }
      }
    };
    // every slice load of a batch is issued, without a branch: past tp a load re-reads the
    // last slice and add_batch drops it (behind a branch each, the later loads waited for
    // earlier ones: measured, deferred TP 10.78 -> 10.50 us at 128 rows)
    {
      // the first slices' loads go out before the fn staging (and a pending call's
      // coefficients) run
      uint4 xv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        xv[u] = load_nt(byte_at(p.xp, row_off + (uint32_t)min(u, p.tp - 1) * slice));
      stage_fn();
      if constexpr (DEFER_IN) finish_pending();
      add_batch(0, xv);
    }
    for (int t0 = 8; t0 < p.tp; t0 += 8) {
      uint4 xv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        xv[u] = load_nt(byte_at(p.xp, row_off + (uint32_t)min(t0 + u, p.tp - 1) * slice));
      __builtin_amdgcn_sched_barrier(0);  // the batch's loads all issue before its sums
      add_batch(t0, xv);
    }
  } else {
    // k ascending, then the shared row
    const uint4 shv = load_nt(byte_at(p.shared, row_off));
    // every gather unconditional (a slot past top_k or out of range reads row 0 with weight
    // 0, and only slots below top_k are added): a gather behind a branch made the compiler
    // wait for every earlier load before issuing the first one
    // no instruction crosses this point, so the gather addresses (each waiting for its slot)
    // are not computed ahead of the loads above, which then stay in flight during that wait
    __builtin_amdgcn_sched_barrier(0);
    uint4 gv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const bool ok = pk[u] >= 0 && pk[u] < p.num_permuted;
      gv[u] = load_nt(byte_at(p.g, ((uint32_t)(ok ? pk[u] : 0) * p.hv + va) * 16u));
      if (!ok) wk[u] = 0.f;
    }
    stage_fn();
    if constexpr (DEFER_IN) finish_pending();
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (u < p.top_k) {
        float f[8];
        unpack8(gv[u], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = __builtin_fmaf(wk[u], f[e], x[e]);
      }
    }
    for (int k = 8; k < p.top_k; ++k) {  // slots beyond 8, in order
      const int pi = *byte_at(p.idx, ((uint32_t)rl * p.top_k + k) * 4u);
      const bool ok = pi >= 0 && pi < p.num_permuted;
      const float w = ok ? *byte_at(p.ew, ((uint32_t)rl * p.top_k + k) * 4u) : 0.f;
      const uint4 gk = load_nt(byte_at(p.g, ((uint32_t)(ok ? pi : 0) * p.hv + va) * 16u));
      float f[8];
      unpack8(gk, f);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = __builtin_fmaf(w, f[e], x[e]);
    }
    float f[8];
    unpack8(shv, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] += f[e];
  }
  round8_bf16(x);  // the reduced output is a bf16 tensor

  // --- new streams (stored at once, and into LDS for the projection), collapse
  const float pst[kN] = {pst4.x, pst4.y, pst4.z, pst4.w};
  const float cmb[kN * kN] = {cmb4[0].x, cmb4[0].y, cmb4[0].z, cmb4[0].w,
                              cmb4[1].x, cmb4[1].y, cmb4[1].z, cmb4[1].w,
                              cmb4[2].x, cmb4[2].y, cmb4[2].z, cmb4[2].w,
                              cmb4[3].x, cmb4[3].y, cmb4[3].z, cmb4[3].w};
  const float pr[kN] = {pr4.x, pr4.y, pr4.z, pr4.w};
  float s[kN][8], sn[kN][8];
#pragma unroll
  for (int j = 0; j < kN; ++j) unpack8(sv[j], s[j]);
  const uint32_t out_off = ((uint32_t)rl * kN * p.hv + va) * 16u;
  float vsq = 0.f;
#pragma unroll
  for (int i = 0; i < kN; ++i) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float a = pst[i] * x[e];
#pragma unroll
      for (int j = 0; j < kN; ++j) a = __builtin_fmaf(cmb[i * kN + j], s[j][e], a);
      sn[i][e] = a;
    }
    const uint4 o = pack8_round(sn[i]);
    if (active) store_nt(byte_at(p.res_out, out_off + (uint32_t)i * p.hv * 16u), o);
    S.sT[i][m][vl] = active ? o : make_uint4(0u, 0u, 0u, 0u);
    unpack8(o, sn[i]);
#pragma unroll
    for (int e = 0; e < 8; ++e) vsq = __builtin_fmaf(sn[i][e], sn[i][e], vsq);
  }
  float y[8];
  float sq = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float a = 0.f;
#pragma unroll
    for (int j = 0; j < kN; ++j) a = __builtin_fmaf(pr[j], sn[j][e], a);
    y[e] = a;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) sq = __builtin_fmaf(y[e], y[e], sq);
  if (!active) {
    sq = 0.f;
    vsq = 0.f;
  }
  sq = half_wave_sum(sq);
  vsq = half_wave_sum(vsq);
  if (vl == 0) {
    S.rowsum[m][0] = sq;
    S.rowsum[m][1] = vsq;
  }

  if (tid < kTileRows) {
    S.want[tid] = epoch_now + 1u;
    S.poisoned[tid] = (unsigned)(ew >> 32);
  }
  __syncthreads();  // fnT, sT, rowsum and want complete

  // --- the rows' sums of y^2 go out first (the handoff waits for them)
  if (tid < kTileRows && row0 + tid < p.rows)
    __hip_atomic_store(word_at(p, ysq_index(p, tile, c, tid)), tagged(S.want[tid], S.rowsum[tid][0]),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // --- partial logits: wave w takes elements 32w .. 32w + 31 of the chunk for all 16 rows;
  // lane (row mm, group kg) holds the MFMA operands of 8 of them
  {
    const int mm = lane & 15, kg = lane >> 4;
    const int hg = wave * 4 + kg;  // vector of the chunk
    f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    // logits 16..31, of which 24..31 are zero: the load reads a row that exists and the
    // value is masked, so it stays an LDS read (a select between the LDS row and a zero in
    // a local variable compiled to a generic load from either place, whose wait then also
    // waited for every store the wave had in flight)
    const bool hi_ok = 16 + mm < kCoefNC;
    const uint32_t keep = hi_ok ? ~0u : 0u;
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int kl = i * kTileH + hg * 8;
      const uint4 a0 = *reinterpret_cast<const uint4*>(&S.fnT[mm][kl]);
      uint4 a1 = *reinterpret_cast<const uint4*>(&S.fnT[hi_ok ? 16 + mm : mm][kl]);
      a1.x &= keep;
      a1.y &= keep;
      a1.z &= keep;
      a1.w &= keep;
      const bf16x8_t b = __builtin_bit_cast(bf16x8_t, S.sT[i][mm][hg]);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a0), b, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a1), b, acc1, 0, 0, 0);
    }
    // D layout: lane holds D[4 kg + i][mm]: logit 4 kg + i (+16) of row mm
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      S.red[wave][mm][4 * kg + i] = acc0[i];
      if (kg < 2) S.red[wave][mm][16 + 4 * kg + i] = acc1[i];
    }
  }

  __syncthreads();  // red complete
  // --- the coefficient partials of this chunk (waves added in order), out before the
  // handoff wait so that they travel while it runs; deferred: as plain floats, in the split
  // layout of the coefficient epilogue (coeff_part_index, split = chunk, splits padded to a
  // multiple of 4 with zeros that chunk 0 writes), read after this kernel has completed
  if (DEFER_OUT && tid < kTileRows * kCoefPartW) {
    const int rr = tid / kCoefPartW, vv = tid % kCoefPartW;
    if (row0 + rr < p.rows) {
      float t = 0.f;
      if (vv < kCoefNC) {
#pragma unroll
        for (int w = 0; w < kTileWaves; ++w) t += S.red[w][rr][vv];
      } else {
        t = S.rowsum[rr][1];
      }
      const int ks = (p.chunks + 3) & ~3;
      const int row = row0 + rr;
      *byte_at(p.part_out, (uint32_t)coeff_part_index(row, vv, c, ks) * 4u) = t;
      if (c == 0)
        for (int z = p.chunks; z < ks; ++z)
          *byte_at(p.part_out, (uint32_t)coeff_part_index(row, vv, z, ks) * 4u) = 0.f;
    }
  }
  if (!DEFER_OUT && tid < kTileRows * kCoefPartW) {
    const int rr = tid / kCoefPartW, vv = tid % kCoefPartW;
    if (row0 + rr < p.rows) {
      float t = 0.f;
      if (vv < kCoefNC) {
#pragma unroll
        for (int w = 0; w < kTileWaves; ++w) t += S.red[w][rr][vv];
      } else {
        t = S.rowsum[rr][1];
      }
      __hip_atomic_store(word_at(p, coef_index(p, tile, c, rr, vv)), tagged(S.want[rr], t),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // --- each half wave: its row's sum of y^2 over every chunk (lane l reads chunk l's word;
  // chunks <= 32), added in a fixed tree order
  float inv;
  {
    const int cl = vl < p.chunks ? vl : p.chunks - 1;  // lanes past the chunks repeat the last
    float part = 0.f;
    bool failed = S.poisoned[m] != 0;
    if (row_ok && !failed) {
      const unsigned want = S.want[m];
      unsigned long long w = 0;
      for (int spins = 0;; ++spins) {
        w = __hip_atomic_load(word_at(p, ysq_index(p, tile, cl, m)), __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
        if ((unsigned)(w >> 32) == want) break;
        if (spins >= p.spin_limit) {
          __hip_atomic_fetch_add(p.errors, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          failed = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      part = vl < p.chunks ? __uint_as_float((unsigned)w) : 0.f;
    }
    float tot = half_wave_sum(part);
    // a wait of this row (half wave) that gave up makes its share of the layer input NaN
    // (and its MXFP8 scales the E8M0 NaN byte)
    const unsigned long long gave_up = __ballot(failed);
    if (((lane < 32) ? (gave_up & 0xFFFFFFFFull) : (gave_up >> 32)) != 0) {
      tot = __builtin_nanf("");
      if (vl == 0 && row_ok && S.poisoned[m] == 0)
        __hip_atomic_store(p.epoch + (size_t)r * kEpochStride + 1, 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    inv = fast_rsq(tot * fast_rcp((float)(p.hv * 8)) + p.eps);
    if (c == 0 && row_ok && vl == 0)
      __hip_atomic_store(p.epoch + (size_t)r * kEpochStride, S.want[m], __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }

  // --- the next coefficients of rows c, c + chunks, ... (row j on wave j % 8), before that
  // wave's layer-input stores so that its wait for the words does not wait for them; lane
  // L < 25 adds value L of every chunk in chunk order
  int j = 0;
  for (int rt = c; !DEFER_OUT && rt < kTileRows; rt += p.chunks, ++j) {
    if (j % kTileWaves != wave) continue;  // wave-uniform
    const int rc = row0 + rt;
    if (rc >= p.rows) continue;
    const unsigned want = S.want[rt];
    float acc = 0.f;
    bool failed = S.poisoned[rt] != 0;
    if (lane < kCoefPartW && !failed) {
      for (int spins = 0;; ++spins) {
        bool ok = true;
        acc = 0.f;
        for (int b0 = 0; b0 < p.chunks; b0 += kFinishBatch) {  // one batch up to 32 chunks
          unsigned long long w[kFinishBatch];
#pragma unroll
          for (int u = 0; u < kFinishBatch; ++u) {
            const int cc = b0 + u < p.chunks ? b0 + u : p.chunks - 1;
            w[u] = __hip_atomic_load(word_at(p, coef_index(p, tile, cc, rt, lane)),
                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
#pragma unroll
          for (int u = 0; u < kFinishBatch; ++u) {
            if (b0 + u < p.chunks) {
              ok = ok && (unsigned)(w[u] >> 32) == want;
              acc += __uint_as_float((unsigned)w[u]);
            }
          }
        }
        if (ok) break;
        if (spins >= p.spin_limit) {
          __hip_atomic_fetch_add(p.errors, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          failed = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    // a wait that gave up makes the row's next coefficients NaN and marks the row
    if (__ballot(failed) != 0) {
      acc = __builtin_nanf("");
      if (lane == 0 && S.poisoned[rt] == 0)
        __hip_atomic_store(p.epoch + (size_t)rc * kEpochStride + 1, 1u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    int slot;
    const float val = coeff_from_sums(coef, lane, acc, sc_l, base_l, &slot);
    if (slot >= 0 && slot < kN) p.next_pre[rc * kN + slot] = val;
    else if (slot >= kN && slot < 2 * kN) p.next_post[rc * kN + slot - kN] = val;
    else if (slot >= 2 * kN) p.next_comb[rc * kN * kN + slot - 2 * kN] = val;
  }

  // --- layer input (and MXFP8)
  {
    float w[8], o[8];
    unpack8(wv, w);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (y[e] * inv) * w[e];
    const uint4 ob = pack8_round(o);
    if (active) store_nt(byte_at(p.layer_out, ((uint32_t)r * p.hv + v) * 16u), ob);
    if constexpr (MXFP8) {
      // 32-element block = the quad of lanes holding vectors v & ~3 .. v | 3
      float q[8];
      unpack8(ob, q);
      float amax = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(q[e]));
      amax = fmaxf(amax, dpp_f32<kDppQuadXor1>(amax));
      amax = fmaxf(amax, dpp_f32<kDppQuadXor2>(amax));
      const int ex = e8m0_exponent(__float_as_uint(amax));
      const float sc = __uint_as_float((uint32_t)(127 - ex) << 23);
      const uint32_t lo = cvt_pk4_e4m3(q[0] * sc, q[1] * sc, q[2] * sc, q[3] * sc);
      const uint32_t hi = cvt_pk4_e4m3(q[4] * sc, q[5] * sc, q[6] * sc, q[7] * sc);
      if (active) {
        store_nt(byte_at(p.mx_data, ((uint32_t)r * p.hv + v) * 8u), make_uint2(lo, hi));
        if ((v & 3) == 0)
          p.mx_scale[mx_scale_offset(r, v >> 2, p.hv / 4, p.scale_kt)] =
              inv == inv ? (uint8_t)(ex + 127) : (uint8_t)0xFF;  // NaN: a wait gave up
      }
    }
  }

  // --- DEFER_IN: the pending call's outputs of this row (lane vl: slot vl), from LDS
  if constexpr (DEFER_IN) {
    if (c == 0 && row_ok && vl < kCoefNC) {
      const float val = reinterpret_cast<const float*>(&S.cf[m][0])[vl];
      if (vl < kN) const_cast<float*>(&p.pre[r].x)[vl] = val;
      else if (vl < 2 * kN) const_cast<float*>(&p.post[r].x)[vl - kN] = val;
      else const_cast<float*>(&p.comb[r * kN].x)[vl - 2 * kN] = val;
    }
  }
}

// DEFER 0 or 1: the argument block is TileParams alone (256 bytes; a larger one costs
// launch time). DEFER 2 takes the pending call's arguments as well (Extra = TileDeferIn).
// One kernel template holds the body: with the body in a device function that two kernels
// call, the compiler's allocation of the DEFER 0 kernels took 40 to 50 more scalar spills.
template <bool FINALIZE, bool MXFP8, int DEFER, typename... Extra>
__global__ __launch_bounds__(kTileThreads, 2) void boundary_tile_kernel(const TileParams p,
                                                                        const Extra... d) {
  prefetch_kernargs<sizeof(TileParams) + (0 + ... + sizeof(Extra))>();
  const TileDeferIn* din = nullptr;
  if constexpr (sizeof...(Extra) > 0) ((din = &d), ...);

  __shared__ __attribute__((aligned(16))) TileShared S;
  // the coefficient epilogue's arguments (kept out of the kernel argument block, which
  // stays within 256 bytes)
  CoeffEpilogue coef;
  coef.part = nullptr;
  coef.ks_count = 0;
  coef.scale = p.scale;
  coef.base = p.base;
  coef.K = kN * p.hv * 8;
  coef.rms_eps = p.rms_eps;
  coef.pre_eps = p.pre_eps;
  coef.sk_eps = p.sk_eps;
  coef.alpha = p.alpha;
  coef.iters = p.iters;
  float sc_l, base_l;
  coeff_lane_scale_base(coef, threadIdx.x & (kWave - 1), &sc_l, &base_l);
  float dsc_l = 0.f, dbase_l = 0.f;  // the pending call's, by lane of the half wave
  if constexpr (DEFER == 2) coeff_lane_scale_base(din->coef, threadIdx.x & 31, &dsc_l, &dbase_l);
  const int wg = blockIdx.x;
  const int xcd = wg % kXcd;
  const int local = wg / kXcd;
  // Placement, in one body for both layouts (uniform selects, not two inlined copies):
  //  groups == 0: a tile's chunks on one XCD, tiles dealt to the XCDs: chunk local % chunks,
  //    tile (round * tiles_per_round + local / chunks) * 8 + xcd;
  //  groups > 0: chunk c of every tile on XCD c % 8 (each XCD reads the fn rows of its own
  //    chunks only): chunk xcd + 8 * (local % groups), tile round * tiles_per_round +
  //    local / groups.
  const bool spread = p.groups != 0;
  const int per = spread ? p.groups : p.chunks;
  const int c = (spread ? xcd : 0) + (spread ? kXcd : 1) * (local % per);
  const int jt = local / per;        // which tile of the round
  if (c >= p.chunks) return;         // past the last chunk (spread only): in no handoff
  const int tile_mul = spread ? 1 : kXcd, tile_add = spread ? 0 : xcd;
  for (int round = 0; round < p.rounds; ++round) {
    const int tile = (round * p.tiles_per_round + jt) * tile_mul + tile_add;
    if (tile * kTileRows >= p.rows) break;  // uniform per workgroup; later rounds go higher
    if (round > 0) __syncthreads();          // LDS reused
    tile_item<FINALIZE, MXFP8, DEFER>(p, coef, din, tile, c, S, sc_l, base_l, dsc_l, dbase_l);
  }
}

template <bool FIN, bool MX, int DEFER>
int occupancy_tile() {
  int n = 0;
  hipError_t e;
  if constexpr (DEFER == 2)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &n, boundary_tile_kernel<FIN, MX, 2, TileDeferIn>, kTileThreads, 0);
  else
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, boundary_tile_kernel<FIN, MX, DEFER>,
                                                     kTileThreads, 0);
  return e == hipSuccess ? n : 0;
}

template <bool FIN, bool MX>
void launch_tile(const TileParams& p, const TileDeferIn* din, int defer, int grid,
                 hipStream_t stream) {
  if (defer == 2)
    hipLaunchKernelGGL((boundary_tile_kernel<FIN, MX, 2, TileDeferIn>), dim3(grid),
                       dim3(kTileThreads), 0, stream, p, *din);
  else if (defer == 1)
    hipLaunchKernelGGL((boundary_tile_kernel<FIN, MX, 1>), dim3(grid), dim3(kTileThreads), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((boundary_tile_kernel<FIN, MX, 0>), dim3(grid), dim3(kTileThreads), 0,
                       stream, p);
}

template <int DEFER>
int occupancy_tile_all() {
  int n = occupancy_tile<false, false, DEFER>();
  n = min(n, occupancy_tile<false, true, DEFER>());
  n = min(n, occupancy_tile<true, false, DEFER>());
  return min(n, occupancy_tile<true, true, DEFER>());
}

}  // namespace

int boundary_tile_resident_wgs_per_cu() {
  return min(occupancy_tile_all<0>(), min(occupancy_tile_all<1>(), occupancy_tile_all<2>()));
}

int boundary_tile_part_ks(int hidden) { return (boundary_tile_chunks(hidden) + 3) & ~3; }

int boundary_tile_chunks(int hidden) { return (hidden + kTileH - 1) / kTileH; }

size_t boundary_tile_words(int rows, int hidden) {
  const size_t tiles = (rows + kTileRows - 1) / kTileRows;
  return tiles * kTileRows * kWordsPerRow * boundary_tile_chunks(hidden);
}

bool boundary_tile_fits(int hidden, int wgs_per_xcd) {
  const int chunks = boundary_tile_chunks(hidden);
  return chunks <= kFinishBatch && chunks <= wgs_per_xcd;
}

hipError_t launch_boundary_tile(const TileLaunch& T, hipStream_t stream) {
  const BoundaryLaunch& L = T.b;
  TileParams p;
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
  p.post = reinterpret_cast<const float4*>(L.post);
  p.comb = reinterpret_cast<const float4*>(L.comb);
  p.pre = reinterpret_cast<const float4*>(L.pre);
  p.norm_w = reinterpret_cast<const uint4*>(L.norm_weight);
  p.eps = L.eps;
  p.rows = L.rows;
  p.hv = L.hidden / 8;
  p.chunks = boundary_tile_chunks(L.hidden);
  p.layer_out = reinterpret_cast<uint4*>(L.layer_input_out);
  p.mx_data = reinterpret_cast<uint2*>(L.mx_data_out);
  p.mx_scale = L.mx_scale_out;
  p.scale_kt = L.scale_kt;
  p.fn = reinterpret_cast<const uint4*>(T.fn);
  p.scale = T.coef.scale;
  p.base = T.coef.base;
  p.rms_eps = T.coef.rms_eps;
  p.pre_eps = T.coef.pre_eps;
  p.sk_eps = T.coef.sk_eps;
  p.alpha = T.coef.alpha;
  p.iters = T.coef.iters;
  const bool defer_out = T.part_out != nullptr;
  if (defer_out)
    p.part_out = T.part_out;
  else
    p.next_pre = T.next_pre;
  p.next_post = T.next_post;
  p.next_comb = T.next_comb;
  p.words = T.words;
  p.epoch = L.epoch;
  p.errors = L.errors;
  p.spin_limit = L.spin_limit;
  if (!boundary_tile_fits(L.hidden, T.wgs_per_xcd)) return hipErrorInvalidConfiguration;
  const int tiles = (L.rows + kTileRows - 1) / kTileRows;
  p.tile_cap = (T.tile_rows + kTileRows - 1) / kTileRows;
  if (tiles > p.tile_cap) return hipErrorInvalidConfiguration;
  int grid;
  if (!T.spread) {
    p.groups = 0;
    const int tile_blocks = (tiles + kXcd - 1) / kXcd;  // tiles per XCD in total
    // a round may use half of the XCD's resident workgroups, or all of them where half
    // does not hold one tile
    int per_xcd = T.wgs_per_xcd / 2;
    if (per_xcd < p.chunks) per_xcd = T.wgs_per_xcd;
    int tpr = per_xcd / p.chunks;
    if (tpr > tile_blocks) tpr = tile_blocks;
    p.tiles_per_round = tpr;
    p.rounds = (tile_blocks + tpr - 1) / tpr;
    grid = kXcd * tpr * p.chunks;
  } else {
    // every tile of a round on every XCD, `groups` chunks of it per XCD; a round takes as
    // many tiles as the XCD's resident workgroups hold
    p.groups = (p.chunks + kXcd - 1) / kXcd;
    int tpr = T.wgs_per_xcd / p.groups;
    if (tpr > tiles) tpr = tiles;
    p.tiles_per_round = tpr;
    p.rounds = (tiles + tpr - 1) / tpr;
    grid = kXcd * tpr * p.groups;
  }
  const bool fin = L.gemm2_permuted != nullptr;
  const bool mx = L.mx_data_out != nullptr;
  TileDeferIn din;
  din.coef = T.in_coef;
  const int defer = T.defer_in ? 2 : (defer_out ? 1 : 0);
  if (T.defer_in && (!defer_out || T.in_coef.ks_count < 4 || T.in_coef.ks_count > kFinishBatch ||
                     T.in_coef.ks_count % 4 != 0))
    return hipErrorInvalidConfiguration;
  if (fin) mx ? launch_tile<true, true>(p, &din, defer, grid, stream)
              : launch_tile<true, false>(p, &din, defer, grid, stream);
  else mx ? launch_tile<false, true>(p, &din, defer, grid, stream)
          : launch_tile<false, false>(p, &din, defer, grid, stream);
  return hipGetLastError();
}

}  // namespace mhc
