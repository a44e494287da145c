// C ABI of libmhc_amd.so: handle lifetime, argument validation and launches.
// The contract of every entry point is stated in include/mhc.h.
#include "mhc.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <new>

#include "kernels.h"

namespace {

constexpr int kHcMult = 4;
constexpr int kMaxRows = 65536;
constexpr int kMaxTp = 64;
constexpr int kMaxTopK = 64;
constexpr int kMaxSinkhornIters = 1000;
constexpr int kDefaultBlock = 128;   // up to kSmallRows rows
constexpr int kManyRowsBlock = 256;
constexpr int kSmallRows = 32;
// Fewer elements per lane pay while the call has few waves per SIMD (measured at hidden
// 7168, boundary + MXFP8: 8 rows 4.90 against 5.29 us, 128 rows 8.72 against 8.83); above
// this many rows the arithmetic is hidden by other waves and the extra waves cost (256
// rows 16.74 against 16.41, 512 rows 29.30 against 28.93)
constexpr int kNarrowMaxRows = 128;
constexpr int kMaxChunks = 64;      // one polling lane per chunk
constexpr int kMaxHidden = 65536;   // chunks per row at the largest block stay <= one wave
constexpr int kDefaultSpinLimit = 1 << 20;
constexpr int kTileMaxRows = 1024;  // rows of the fused boundary + coefficient scratch

}  // namespace

struct mhc_ctx {
  int hidden, hc_mult, max_rows, max_tp, top_k, device;
  int slot_stride;         // handoff words per row (chunks at the smallest block, padded)
  int block;               // layer-input workgroup size for up to kSmallRows rows (auto)
  int block_many;          // ... for more rows (auto)
  int block_set;           // the size MHC_OPT_BOUNDARY_BLOCK set, 0: automatic
  int spin_limit;          // polls before a handoff wait gives up
  bool xcd_available;      // the probe at creation found workgroup ids dealt round-robin
                           // to the XCDs
  bool xcd_handoff;        // a row's handoff words go through its XCD's L2 (else device
                           // scope): MHC_OPT_ROW_HANDOFF
  int scale_layout;        // MHC_SCALE_ROW_MAJOR or MHC_SCALE_SWIZZLED_128X4
  int tile_placement;      // MHC_TILE_PER_XCD or MHC_TILE_SPREAD (the fused kernel)
  int lane_elems;          // the fewest elements per lane the layer-input kernels may use
                           // (2, 4 or 8; fewer run at more threads: the same chunks per row)
  int wgs_per_xcd[3];      // resident layer-input workgroups per XCD at block 128 / 256 / 512
  int tile_wgs_per_xcd;    // resident workgroups of the fused boundary + coefficient kernel
  int tile_rows;           // rows the fused kernel's scratch covers (0: not available)
  size_t pre_floats;       // coefficient-path scratch
  void* scratch;           // one allocation: slots | epoch | errors | tile_words | pre_part
  unsigned long long* slots;
  float* pre_part;
  unsigned* epoch;
  unsigned* errors;
  unsigned long long* tile_words;  // the fused kernel's tagged partials
  float* tile_part[2];     // a deferred fused call's coefficient partials (used in turn)
  int tile_part_next;      // the buffer the next deferred fused call writes
  size_t zero_words;       // 32-bit words up to pre_part (cleared by mhc_reset)
  // a deferred coefficient call whose epilogue has not been enqueued yet
  bool pending;
  mhc::PreLaunch pend;
};

namespace {

inline int block_index(int block) {
  return block == 128 ? 0 : (block == 256 ? 1 : (block == 512 ? 2 : -1));
}

// Whether a handle may run the boundary at this block size: a row's chunks fit the
// polling wave and half of an XCD's resident workgroups (a launch then spans rows
// in rounds of at most half of the XCD).
inline bool block_usable(const mhc_ctx* h, int block) {
  const int i = block_index(block);
  if (i < 0) return false;
  const int chunks = mhc::boundary_chunks(h->hidden, block);
  return chunks <= kMaxChunks && h->wgs_per_xcd[i] / 2 >= chunks;
}

inline bool aligned(const void* p, unsigned a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int check_device(const mhc_ctx* h) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return MHC_ERR_HIP;
  return cur == h->device ? MHC_OK : MHC_ERR_DEVICE;
}

inline int launch_status(hipError_t e) { return e == hipSuccess ? MHC_OK : MHC_ERR_HIP; }

// Common validation of the mHC half of a boundary call (streams, mixes, pre,
// norm, outputs). Returns MHC_OK or the first failing status.
int check_mix(const mhc_ctx* h, const uint16_t* residual, const float* post, const float* comb,
              const float* pre, const uint16_t* norm_weight, float norm_eps, uint16_t* residual_out,
              uint16_t* layer_input_out, uint8_t* mx_data_out, uint8_t* mx_scale_out) {
  if (!residual || !post || !comb || !residual_out) return MHC_ERR_INVALID_ARG;
  const bool has_pre = pre != nullptr;
  if (has_pre != (norm_weight != nullptr) || has_pre != (layer_input_out != nullptr))
    return MHC_ERR_INVALID_ARG;
  if ((mx_data_out == nullptr) != (mx_scale_out == nullptr)) return MHC_ERR_INVALID_ARG;
  if (mx_data_out && !has_pre) return MHC_ERR_INVALID_ARG;
  if (mx_data_out && (h->hidden % 32) != 0) return MHC_ERR_UNSUPPORTED;
  if (has_pre && !(norm_eps >= 0.0f)) return MHC_ERR_SHAPE;  // also rejects NaN
  if (!aligned(residual, 16) || !aligned(residual_out, 16) || !aligned(post, 4) ||
      !aligned(comb, 4))
    return MHC_ERR_ALIGN;
  if (has_pre && (!aligned(pre, 4) || !aligned(norm_weight, 16) || !aligned(layer_input_out, 16)))
    return MHC_ERR_ALIGN;
  if (mx_data_out && !aligned(mx_data_out, 8)) return MHC_ERR_ALIGN;
  return MHC_OK;
}

void fill_mix(const mhc_ctx* h, mhc::BoundaryLaunch& L, const uint16_t* residual,
              const float* post, const float* comb, const float* pre, const uint16_t* norm_weight,
              float norm_eps, int rows, uint16_t* residual_out, uint16_t* layer_input_out,
              uint8_t* mx_data_out, uint8_t* mx_scale_out) {
  L.residual = residual;
  L.residual_out = residual_out;
  L.post = post;
  L.comb = comb;
  L.pre = pre;
  L.norm_weight = norm_weight;
  L.eps = norm_eps;
  L.rows = rows;
  L.hidden = h->hidden;
  L.layer_input_out = layer_input_out;
  L.mx_data_out = mx_data_out;
  L.mx_scale_out = mx_scale_out;
  L.scale_kt = h->scale_layout == MHC_SCALE_SWIZZLED_128X4 ? (h->hidden / 32 + 3) / 4 : 0;
  L.slots = h->slots;
  L.epoch = h->epoch;
  L.errors = h->errors;
  L.slot_stride = h->slot_stride;
  L.spin_limit = h->spin_limit;
  L.xcd_handoff = h->xcd_handoff;
  const int block = h->block_set ? h->block_set : (rows > kSmallRows ? h->block_many : h->block);
  L.max_wgs_per_xcd = h->wgs_per_xcd[block_index(block)];
  L.block = block;
  // the narrower forms (2 or 4 elements per lane): 8 / elements times the threads, the same
  // chunks per row; the fewest elements allowed whose workgroup size exists and still fits
  // a row in half an XCD (used by the kernels that have them)
  L.lane_elems = 8;
  L.block_n = 0;
  L.max_wgs_per_xcd_n = 0;
  for (int el = h->lane_elems; el < 8 && !h->block_set && rows <= kNarrowMaxRows; el *= 2) {
    const int bn = block * (8 / el);
    if (block_index(bn) < 0) continue;
    const int wn = h->wgs_per_xcd[block_index(bn)];
    if (wn / 2 < mhc::boundary_chunks(h->hidden, block)) continue;
    L.lane_elems = el;
    L.block_n = bn;
    L.max_wgs_per_xcd_n = wn;
    break;
  }
}

// Enqueue the epilogue of a pending deferred coefficient call, if any.
int flush_pending(mhc_ctx* h, hipStream_t stream) {
  if (!h->pending) return MHC_OK;
  h->pending = false;
  return launch_status(mhc::launch_pre_epilogue(h->pend, stream));
}

// A boundary call that consumes the pending call's outputs finishes its epilogue in the
// kernel; any other boundary call enqueues the epilogue first.
int take_pending(mhc_ctx* h, mhc::BoundaryLaunch& L, const float* post, const float* comb,
                 const float* pre, int rows, hipStream_t stream) {
  if (!h->pending) return MHC_OK;
  const bool match = post == h->pend.post_out && comb == h->pend.comb_out &&
                     (pre == nullptr || pre == h->pend.pre_out) && rows == h->pend.rows;
  if (!match) return flush_pending(h, stream);
  h->pending = false;
  L.defer = true;
  L.coef = mhc::pre_epilogue_args(h->pend);
  L.pre_pending = h->pend.pre_out;
  return MHC_OK;
}

}  // namespace

namespace mhc {

__global__ void fill_u32_kernel(unsigned* p, size_t n, unsigned value) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = value;
}

hipError_t launch_fill_u32(unsigned* p, size_t n, unsigned value, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int grid = (int)((n + 255) / 256);
  hipLaunchKernelGGL(fill_u32_kernel, dim3(grid), dim3(256), 0, stream, p, n, value);
  return hipGetLastError();
}

}  // namespace mhc

// ---------------------------------------------------------------------------
// The allocation-free boundary (mhc_boundary_noalloc): the row handoff's words, epochs and
// error word live in a fixed array in device memory, one copy per GPU, instead of a
// handle's hipMalloc. Its size bounds the rows (1 KiB of words, one per wave of the row,
// and one 128-byte line of epochs per row) and the hidden size (at most 16384, i.e. 128
// waves per row at 512 threads).
// ---------------------------------------------------------------------------
namespace {

constexpr int kNoAllocRows = 1024;
constexpr int kNoAllocSlotStride = 128;  // boundary_handoff_words(kNoAllocMaxHidden)
constexpr int kNoAllocMaxHidden = 16384;
constexpr size_t kNoAllocSlotBytes = (size_t)kNoAllocRows * kNoAllocSlotStride * 8;
constexpr size_t kNoAllocEpochBytes = (size_t)kNoAllocRows * mhc::kEpochStride * 4;
constexpr size_t kNoAllocBytes = kNoAllocSlotBytes + kNoAllocEpochBytes + 256;
constexpr int kNoAllocMaxDevices = 64;

struct NoAllocDevice {
  std::atomic<int> ready;  // set-up done on this device
  char* scratch;           // this device's copy of `scratch` (from hipGetSymbolAddress)
  int wgs_per_xcd[3];      // resident layer-input workgroups per XCD at 128 / 256 / 512
};
NoAllocDevice g_noalloc[kNoAllocMaxDevices];
std::mutex g_noalloc_mu;

}  // namespace

// In host code this name stands for the array but is not its device address: kernels and
// fills get the address each device reports at set-up.
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

namespace {

// Once per device, with that device current: the array's address on it, the kernels'
// occupancy there, and the array zeroed on `stream` before the first call's kernels.
int noalloc_setup(int dev, hipStream_t stream, NoAllocDevice** out) {
  if (dev < 0 || dev >= kNoAllocMaxDevices) return MHC_ERR_UNSUPPORTED;
  NoAllocDevice& d = g_noalloc[dev];
  if (d.ready.load(std::memory_order_acquire) == 0) {
    std::lock_guard<std::mutex> lock(g_noalloc_mu);
    if (d.ready.load(std::memory_order_relaxed) == 0) {
      void* ptr = nullptr;
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
        return MHC_ERR_HIP;
      int cus = 0;
      if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
              hipSuccess ||
          cus < 8)
        return MHC_ERR_HIP;
      const int blocks[3] = {128, 256, 512};
      for (int i = 0; i < 3; ++i)
        d.wgs_per_xcd[i] = mhc::boundary_resident_wgs_per_cu(blocks[i]) * (cus / 8);
      if (mhc::launch_fill_u32(static_cast<unsigned*>(ptr), kNoAllocBytes / 4, 0u, stream) !=
          hipSuccess)
        return MHC_ERR_HIP;
      d.scratch = static_cast<char*>(ptr);
      d.ready.store(1, std::memory_order_release);
    }
  }
  *out = &d;
  return MHC_OK;
}

}  // namespace

extern "C" {

const char* mhc_status_string(int status) {
  switch (status) {
    case MHC_OK: return "MHC_OK";
    case MHC_ERR_INVALID_ARG: return "MHC_ERR_INVALID_ARG: null or inconsistent argument";
    case MHC_ERR_SHAPE: return "MHC_ERR_SHAPE: invalid size";
    case MHC_ERR_ALIGN: return "MHC_ERR_ALIGN: misaligned pointer";
    case MHC_ERR_LIMIT:
      return "MHC_ERR_LIMIT: rows, tp or hidden above the limit (the handle's, or the "
             "allocation-free call's fixed scratch)";
    case MHC_ERR_UNSUPPORTED: return "MHC_ERR_UNSUPPORTED: unsupported configuration";
    case MHC_ERR_HIP: return "MHC_ERR_HIP: HIP runtime call failed";
    case MHC_ERR_DEVICE: return "MHC_ERR_DEVICE: current device is not the handle's device";
    default: return "MHC: unknown status";
  }
}

int mhc_create(int hidden, int hc_mult, int max_rows, int max_tp, int top_k, int device,
               mhc_handle* out) {
  if (!out) return MHC_ERR_INVALID_ARG;
  *out = nullptr;
  if (hidden <= 0 || hidden % 8 != 0 || hidden > kMaxHidden) return MHC_ERR_SHAPE;
  if (max_rows < 1 || max_rows > kMaxRows || max_tp < 1 || max_tp > kMaxTp || top_k < 1 ||
      top_k > kMaxTopK || device < 0)
    return MHC_ERR_SHAPE;
  if (hc_mult != kHcMult) return MHC_ERR_UNSUPPORTED;

  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || device >= ndev) return MHC_ERR_HIP;
  int prev = 0;
  if (hipGetDevice(&prev) != hipSuccess) return MHC_ERR_HIP;
  if (hipSetDevice(device) != hipSuccess) return MHC_ERR_HIP;

  mhc_ctx* h = new (std::nothrow) mhc_ctx();
  if (!h) {
    (void)hipSetDevice(prev);
    return MHC_ERR_HIP;
  }
  h->hidden = hidden;
  h->hc_mult = hc_mult;
  h->max_rows = max_rows;
  h->max_tp = max_tp;
  h->top_k = top_k;
  h->device = device;
  h->block = kDefaultBlock;
  h->spin_limit = kDefaultSpinLimit;
  h->scale_layout = MHC_SCALE_ROW_MAJOR;
  h->lane_elems = 2;
  // chunks spread over the XCDs: each XCD then reads only its chunks' rows of fn, which a
  // decode step reads cold for every sublayer (measured: the fused + deferred step at 128
  // rows 1447 -> 1396 us); a tile per XCD is ahead only when one fn is reused while it
  // is still cached (10.6 against 11.1 us per deferred call)
  h->tile_placement = MHC_TILE_SPREAD;
  h->pending = false;
  // one word per wave of the row at the most waves per row (the smallest chunks at the
  // widest workgroup), rounded up to 16 words: each row's handoff words on 128-byte lines
  // of their own (rows sharing a line, from different XCDs, measured 0.25 us slower per
  // call: 5.35 against 5.08 us for 32 rows at hidden 7168)
  h->slot_stride = mhc::boundary_handoff_words(hidden);
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
      cus < 8) {
    delete h;
    (void)hipSetDevice(prev);
    return MHC_ERR_HIP;
  }
  const int blocks[3] = {128, 256, 512};
  for (int i = 0; i < 3; ++i)
    h->wgs_per_xcd[i] = mhc::boundary_resident_wgs_per_cu(blocks[i]) * (cus / 8);
  h->block = 0;
  for (int b : {kDefaultBlock, 256, 512}) {
    if (block_usable(h, b)) {
      h->block = b;
      break;
    }
  }
  if (h->block == 0) {
    delete h;
    (void)hipSetDevice(prev);
    return MHC_ERR_UNSUPPORTED;
  }
  // above kSmallRows rows 256 threads run faster (measured at hidden 7168, 32 to 512 rows)
  h->block_many = block_usable(h, kManyRowsBlock) ? kManyRowsBlock : h->block;
  h->block_set = 0;
  size_t pre_floats = 0;
  for (int r = 1; r <= max_rows; r += 16) {  // the split plan changes only every 16 rows
    const size_t f = mhc::pre_scratch_floats_for(r, hidden);
    if (f > pre_floats) pre_floats = f;
  }
  h->pre_floats = pre_floats;

  h->tile_wgs_per_xcd = mhc::boundary_tile_resident_wgs_per_cu() * (cus / 8);
  h->tile_rows = mhc::boundary_tile_fits(hidden, h->tile_wgs_per_xcd)
                     ? (max_rows < kTileMaxRows ? max_rows : kTileMaxRows)
                     : 0;

  const size_t slot_bytes = round_up((size_t)max_rows * h->slot_stride * 8, 256);
  const size_t epoch_bytes = round_up((size_t)max_rows * mhc::kEpochStride * 4, 256);
  const size_t err_bytes = 256;
  const size_t tile_bytes = round_up(mhc::boundary_tile_words(h->tile_rows, hidden) * 8, 256);
  const size_t pre_bytes = round_up(pre_floats * sizeof(float), 256);
  const size_t part_bytes =
      round_up((size_t)h->tile_rows * 25 * mhc::boundary_tile_part_ks(hidden) * sizeof(float),
               256);
  const size_t total =
      slot_bytes + epoch_bytes + err_bytes + tile_bytes + pre_bytes + 2 * part_bytes;
  void* base = nullptr;
  if (hipMalloc(&base, total) != hipSuccess) {
    delete h;
    (void)hipSetDevice(prev);
    return MHC_ERR_HIP;
  }
  char* b = static_cast<char*>(base);
  h->scratch = base;
  h->slots = reinterpret_cast<unsigned long long*>(b);
  h->epoch = reinterpret_cast<unsigned*>(b + slot_bytes);
  h->errors = reinterpret_cast<unsigned*>(b + slot_bytes + epoch_bytes);
  h->tile_words =
      reinterpret_cast<unsigned long long*>(b + slot_bytes + epoch_bytes + err_bytes);
  h->pre_part =
      reinterpret_cast<float*>(b + slot_bytes + epoch_bytes + err_bytes + tile_bytes);
  char* parts = b + slot_bytes + epoch_bytes + err_bytes + tile_bytes + pre_bytes;
  h->tile_part[0] = reinterpret_cast<float*>(parts);
  h->tile_part[1] = reinterpret_cast<float*>(parts + part_bytes);
  h->tile_part_next = 0;
  h->zero_words = (slot_bytes + epoch_bytes + err_bytes + tile_bytes) / 4;
  // the scratch is far larger than the probe's words; it is zeroed right after
  hipError_t e = hipSuccess;
  h->xcd_available = false;
  if (total >= mhc::kXcdProbeWgs * sizeof(unsigned))
    e = mhc::probe_xcd_round_robin(reinterpret_cast<unsigned*>(base), &h->xcd_available);
  h->xcd_handoff = h->xcd_available;
  if (e == hipSuccess)
    e = mhc::launch_fill_u32(reinterpret_cast<unsigned*>(base), total / 4, 0u, nullptr);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  (void)hipSetDevice(prev);
  if (e != hipSuccess) {
    (void)hipFree(base);
    delete h;
    return MHC_ERR_HIP;
  }
  *out = h;
  return MHC_OK;
}

int mhc_set_option(mhc_handle h, int option, int value) {
  if (!h) return MHC_ERR_INVALID_ARG;
  switch (option) {
    case MHC_OPT_BOUNDARY_BLOCK:
      if (block_index(value) < 0) return MHC_ERR_SHAPE;
      if (!block_usable(h, value)) return MHC_ERR_UNSUPPORTED;
      h->block_set = value;
      return MHC_OK;
    case MHC_OPT_SPIN_LIMIT:
      if (value < 0) return MHC_ERR_SHAPE;
      h->spin_limit = value;
      return MHC_OK;
    case MHC_OPT_LANE_ELEMS:
      if (value != 8 && value != 4 && value != 2) return MHC_ERR_SHAPE;
      h->lane_elems = value;
      return MHC_OK;
    case MHC_OPT_SCALE_LAYOUT:
      if (value != MHC_SCALE_ROW_MAJOR && value != MHC_SCALE_SWIZZLED_128X4) return MHC_ERR_SHAPE;
      h->scale_layout = value;
      return MHC_OK;
    case MHC_OPT_TILE_PLACEMENT:
      if (value != MHC_TILE_PER_XCD && value != MHC_TILE_SPREAD) return MHC_ERR_SHAPE;
      h->tile_placement = value;
      return MHC_OK;
    case MHC_OPT_ROW_HANDOFF:
      if (value != MHC_HANDOFF_DEVICE && value != MHC_HANDOFF_XCD) return MHC_ERR_SHAPE;
      if (value == MHC_HANDOFF_XCD && !h->xcd_available) return MHC_ERR_UNSUPPORTED;
      h->xcd_handoff = value == MHC_HANDOFF_XCD;
      return MHC_OK;
    default:
      return MHC_ERR_INVALID_ARG;
  }
}

int mhc_mxfp8_scale_bytes(int rows, int hidden, int layout, uint64_t* bytes) {
  if (!bytes) return MHC_ERR_INVALID_ARG;
  if (rows < 0 || hidden <= 0 || hidden % 32 != 0) return MHC_ERR_SHAPE;
  const uint64_t blocks = (uint64_t)(hidden / 32);
  switch (layout) {
    case MHC_SCALE_ROW_MAJOR:
      *bytes = (uint64_t)rows * blocks;
      return MHC_OK;
    case MHC_SCALE_SWIZZLED_128X4:
      *bytes = round_up((uint64_t)rows, 128) * round_up(blocks, 4);
      return MHC_OK;
    default:
      return MHC_ERR_SHAPE;
  }
}

int mhc_get_errors(mhc_handle h, unsigned* count, int clear, mhc_stream_t stream) {
  if (!h || !count) return MHC_ERR_INVALID_ARG;
  int st = check_device(h);
  if (st != MHC_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(count, h->errors, sizeof(unsigned), hipMemcpyDeviceToHost, s) != hipSuccess)
    return MHC_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return MHC_ERR_HIP;
  // a count above zero may leave stale handoff words behind: clearing it re-zeroes the
  // whole handoff state, as mhc_reset does
  if (clear)
    return launch_status(mhc::launch_fill_u32(reinterpret_cast<unsigned*>(h->scratch),
                                              h->zero_words, 0u, s));
  return MHC_OK;
}

int mhc_destroy(mhc_handle h) {
  if (!h) return MHC_OK;
  int prev = 0;
  int st = MHC_OK;
  if (hipGetDevice(&prev) != hipSuccess) st = MHC_ERR_HIP;
  if (hipSetDevice(h->device) != hipSuccess) st = MHC_ERR_HIP;
  if (hipDeviceSynchronize() != hipSuccess) st = MHC_ERR_HIP;
  if (hipFree(h->scratch) != hipSuccess) st = MHC_ERR_HIP;
  (void)hipSetDevice(prev);
  delete h;
  return st;
}

int mhc_reset(mhc_handle h, mhc_stream_t stream) {
  if (!h) return MHC_ERR_INVALID_ARG;
  int st = check_device(h);
  if (st != MHC_OK) return st;
  return launch_status(mhc::launch_fill_u32(reinterpret_cast<unsigned*>(h->scratch), h->zero_words,
                                            0u, static_cast<hipStream_t>(stream)));
}

int mhc_boundary(mhc_handle h, const uint16_t* x_partials, int tp, const uint16_t* residual,
                 const float* post, const float* comb, const float* pre,
                 const uint16_t* norm_weight, float norm_eps, int rows, uint16_t* residual_out,
                 uint16_t* layer_input_out, uint8_t* mx_data_out, uint8_t* mx_scale_out,
                 mhc_stream_t stream) {
  if (!h) return MHC_ERR_INVALID_ARG;
  if (rows < 0 || tp < 1) return MHC_ERR_SHAPE;
  if (rows > h->max_rows || tp > h->max_tp) return MHC_ERR_LIMIT;
  if (rows == 0) return MHC_OK;
  if (!x_partials) return MHC_ERR_INVALID_ARG;
  int st = check_mix(h, residual, post, comb, pre, norm_weight, norm_eps, residual_out,
                     layer_input_out, mx_data_out, mx_scale_out);
  if (st != MHC_OK) return st;
  if (!aligned(x_partials, 16)) return MHC_ERR_ALIGN;
  st = check_device(h);
  if (st != MHC_OK) return st;
  mhc::BoundaryLaunch L = {};
  L.x_partials = x_partials;
  L.tp = tp;
  fill_mix(h, L, residual, post, comb, pre, norm_weight, norm_eps, rows, residual_out,
           layer_input_out, mx_data_out, mx_scale_out);
  st = take_pending(h, L, post, comb, pre, rows, static_cast<hipStream_t>(stream));
  if (st != MHC_OK) return st;
  return launch_status(mhc::launch_boundary(L, static_cast<hipStream_t>(stream)));
}

int mhc_boundary_noalloc(int hidden, const uint16_t* x_partials, int tp,
                         const uint16_t* residual, const float* post, const float* comb,
                         const float* pre, const uint16_t* norm_weight, float norm_eps, int rows,
                         uint16_t* residual_out, uint16_t* layer_input_out, uint8_t* mx_data_out,
                         uint8_t* mx_scale_out, int reset, mhc_stream_t stream) {
  if (hidden <= 0 || hidden % 8 != 0 || rows < 0 || tp < 1) return MHC_ERR_SHAPE;
  if (hidden > kNoAllocMaxHidden || rows > kNoAllocRows || tp > kMaxTp) return MHC_ERR_LIMIT;
  if (rows == 0) return MHC_OK;
  if (!x_partials) return MHC_ERR_INVALID_ARG;
  // a context on the stack: the device's set-up and this call's hidden size, with the
  // handle's defaults (automatic block size, two elements per lane, row-major scales)
  mhc_ctx h{};
  h.hidden = hidden;
  h.hc_mult = kHcMult;
  h.max_rows = kNoAllocRows;
  h.max_tp = kMaxTp;
  h.top_k = 1;
  h.slot_stride = kNoAllocSlotStride;
  h.spin_limit = kDefaultSpinLimit;
  h.scale_layout = MHC_SCALE_ROW_MAJOR;
  h.lane_elems = 2;
  int st = check_mix(&h, residual, post, comb, pre, norm_weight, norm_eps, residual_out,
                     layer_input_out, mx_data_out, mx_scale_out);
  if (st != MHC_OK) return st;
  if (!aligned(x_partials, 16)) return MHC_ERR_ALIGN;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MHC_ERR_HIP;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  NoAllocDevice* d = nullptr;
  st = noalloc_setup(dev, s, &d);
  if (st != MHC_OK) return st;
  h.device = dev;
  for (int i = 0; i < 3; ++i) h.wgs_per_xcd[i] = d->wgs_per_xcd[i];
  h.block = 0;
  for (int b : {kDefaultBlock, 256, 512}) {
    if (block_usable(&h, b)) {
      h.block = b;
      break;
    }
  }
  if (h.block == 0) return MHC_ERR_UNSUPPORTED;
  h.block_many = block_usable(&h, kManyRowsBlock) ? kManyRowsBlock : h.block;
  h.slots = reinterpret_cast<unsigned long long*>(d->scratch);
  h.epoch = reinterpret_cast<unsigned*>(d->scratch + kNoAllocSlotBytes);
  h.errors = reinterpret_cast<unsigned*>(d->scratch + kNoAllocSlotBytes + kNoAllocEpochBytes);
  if (reset && mhc::launch_fill_u32(reinterpret_cast<unsigned*>(d->scratch), kNoAllocBytes / 4,
                                    0u, s) != hipSuccess)
    return MHC_ERR_HIP;
  mhc::BoundaryLaunch L = {};
  L.x_partials = x_partials;
  L.tp = tp;
  fill_mix(&h, L, residual, post, comb, pre, norm_weight, norm_eps, rows, residual_out,
           layer_input_out, mx_data_out, mx_scale_out);
  return launch_status(mhc::launch_boundary(L, s));
}

int mhc_residual_only(mhc_handle h, const uint16_t* x_partials, int tp, const uint16_t* residual,
                      const float* post, const float* comb, int rows, uint16_t* residual_out,
                      mhc_stream_t stream) {
  return mhc_boundary(h, x_partials, tp, residual, post, comb, nullptr, nullptr, 0.0f, rows,
                      residual_out, nullptr, nullptr, nullptr, stream);
}

int mhc_finalize(mhc_handle h, const uint16_t* gemm2_permuted, int num_permuted,
                 const float* expert_weights, const int32_t* expanded_idx_to_permuted_idx,
                 const uint16_t* shared_output, const uint16_t* residual, const float* post,
                 const float* comb, const float* pre, const uint16_t* norm_weight, float norm_eps,
                 int rows, uint16_t* residual_out, uint16_t* layer_input_out,
                 uint8_t* mx_data_out, uint8_t* mx_scale_out, mhc_stream_t stream) {
  if (!h) return MHC_ERR_INVALID_ARG;
  if (rows < 0 || num_permuted < 1) return MHC_ERR_SHAPE;
  if (rows > h->max_rows) return MHC_ERR_LIMIT;
  if (rows == 0) return MHC_OK;
  if (!gemm2_permuted || !expert_weights || !expanded_idx_to_permuted_idx || !shared_output)
    return MHC_ERR_INVALID_ARG;
  int st = check_mix(h, residual, post, comb, pre, norm_weight, norm_eps, residual_out,
                     layer_input_out, mx_data_out, mx_scale_out);
  if (st != MHC_OK) return st;
  if (!aligned(gemm2_permuted, 16) || !aligned(shared_output, 16) || !aligned(expert_weights, 4) ||
      !aligned(expanded_idx_to_permuted_idx, 4))
    return MHC_ERR_ALIGN;
  st = check_device(h);
  if (st != MHC_OK) return st;
  mhc::BoundaryLaunch L = {};
  L.gemm2_permuted = gemm2_permuted;
  L.num_permuted = num_permuted;
  L.expert_weights = expert_weights;
  L.idx = expanded_idx_to_permuted_idx;
  L.shared_output = shared_output;
  L.top_k = h->top_k;
  fill_mix(h, L, residual, post, comb, pre, norm_weight, norm_eps, rows, residual_out,
           layer_input_out, mx_data_out, mx_scale_out);
  st = take_pending(h, L, post, comb, pre, rows, static_cast<hipStream_t>(stream));
  if (st != MHC_OK) return st;
  return launch_status(mhc::launch_boundary(L, static_cast<hipStream_t>(stream)));
}

int mhc_first(mhc_handle h, const uint16_t* x, const uint16_t* norm_weight, float norm_eps,
              int rows, uint16_t* residual_out, uint16_t* layer_input_out, uint8_t* mx_data_out,
              uint8_t* mx_scale_out, mhc_stream_t stream) {
  if (!h) return MHC_ERR_INVALID_ARG;
  if (rows < 0) return MHC_ERR_SHAPE;
  if (rows > h->max_rows) return MHC_ERR_LIMIT;
  if (rows == 0) return MHC_OK;
  if (!x || !norm_weight || !residual_out || !layer_input_out) return MHC_ERR_INVALID_ARG;
  if ((mx_data_out == nullptr) != (mx_scale_out == nullptr)) return MHC_ERR_INVALID_ARG;
  if (mx_data_out && (h->hidden % 32) != 0) return MHC_ERR_UNSUPPORTED;
  if (!(norm_eps >= 0.0f)) return MHC_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(norm_weight, 16) || !aligned(residual_out, 16) ||
      !aligned(layer_input_out, 16) || (mx_data_out && !aligned(mx_data_out, 8)))
    return MHC_ERR_ALIGN;
  int st = check_device(h);
  if (st != MHC_OK) return st;
  mhc::BoundaryLaunch L = {};
  st = flush_pending(h, static_cast<hipStream_t>(stream));
  if (st != MHC_OK) return st;
  fill_mix(h, L, nullptr, nullptr, nullptr, nullptr, norm_weight, norm_eps, rows,
           residual_out, layer_input_out, mx_data_out, mx_scale_out);
  L.x_partials = x;
  L.tp = 1;
  L.mode = mhc::kBoundaryFirst;
  return launch_status(mhc::launch_boundary(L, static_cast<hipStream_t>(stream)));
}

int mhc_collapse_norm(mhc_handle h, const uint16_t* residual, const float* pre,
                      const uint16_t* norm_weight, float norm_eps, int rows, uint16_t* out,
                      uint8_t* mx_data_out, uint8_t* mx_scale_out, mhc_stream_t stream) {
  if (!h) return MHC_ERR_INVALID_ARG;
  if (rows < 0) return MHC_ERR_SHAPE;
  if (rows > h->max_rows) return MHC_ERR_LIMIT;
  if (rows == 0) return MHC_OK;
  if (!residual || !pre || !norm_weight || !out) return MHC_ERR_INVALID_ARG;
  if ((mx_data_out == nullptr) != (mx_scale_out == nullptr)) return MHC_ERR_INVALID_ARG;
  if (mx_data_out && (h->hidden % 32) != 0) return MHC_ERR_UNSUPPORTED;
  if (!(norm_eps >= 0.0f)) return MHC_ERR_SHAPE;
  if (!aligned(residual, 16) || !aligned(pre, 4) || !aligned(norm_weight, 16) ||
      !aligned(out, 16) || (mx_data_out && !aligned(mx_data_out, 8)))
    return MHC_ERR_ALIGN;
  int st = check_device(h);
  if (st != MHC_OK) return st;
  mhc::BoundaryLaunch L = {};
  st = flush_pending(h, static_cast<hipStream_t>(stream));
  if (st != MHC_OK) return st;
  fill_mix(h, L, residual, nullptr, nullptr, pre, norm_weight, norm_eps, rows, nullptr,
           out, mx_data_out, mx_scale_out);
  L.mode = mhc::kBoundaryHead;
  return launch_status(mhc::launch_boundary(L, static_cast<hipStream_t>(stream)));
}

int mhc_collapse_mean(mhc_handle h, const uint16_t* streams, int rows, uint16_t* out,
                      mhc_stream_t stream) {
  if (!h) return MHC_ERR_INVALID_ARG;
  if (rows < 0) return MHC_ERR_SHAPE;
  if (rows > h->max_rows) return MHC_ERR_LIMIT;
  if (rows == 0) return MHC_OK;
  if (!streams || !out) return MHC_ERR_INVALID_ARG;
  if (!aligned(streams, 16) || !aligned(out, 16)) return MHC_ERR_ALIGN;
  int st = check_device(h);
  if (st != MHC_OK) return st;
  st = flush_pending(h, static_cast<hipStream_t>(stream));
  if (st != MHC_OK) return st;
  return launch_status(
      mhc::launch_collapse_mean(streams, rows, h->hidden, out, static_cast<hipStream_t>(stream)));
}

namespace {

int check_coeff_args(const mhc_coeff_args* a) {
  if (!a) return MHC_ERR_INVALID_ARG;
  if (a->sinkhorn_iters < 0 || a->sinkhorn_iters > kMaxSinkhornIters) return MHC_ERR_SHAPE;
  if (!(a->rms_eps >= 0.0f) || !(a->sinkhorn_eps >= 0.0f)) return MHC_ERR_SHAPE;
  if (a->deferred != 0 && a->deferred != 1) return MHC_ERR_INVALID_ARG;
  if (!a->fn || !a->scale || !a->base || !a->pre_out || !a->post_out || !a->comb_out)
    return MHC_ERR_INVALID_ARG;
  if (!aligned(a->fn, 16) || !aligned(a->scale, 4) || !aligned(a->base, 4) ||
      !aligned(a->pre_out, 4) || !aligned(a->post_out, 4) || !aligned(a->comb_out, 4))
    return MHC_ERR_ALIGN;
  return MHC_OK;
}

// A boundary followed by the next coefficient call on its new streams: one kernel where
// the fused form applies, else the two calls. L is the boundary's launch, already filled.
int boundary_then_coeffs(mhc_ctx* h, mhc::BoundaryLaunch& L, const mhc_coeff_args* a,
                         hipStream_t s) {
  // (the fused kernel addresses its tensors with 32-bit byte offsets: the gathered MoE rows
  // must stay below 4 GiB; the others do within its row and hidden limits)
  const bool fused = h->tile_rows >= L.rows && aligned(L.post, 16) && aligned(L.comb, 16) &&
                     aligned(L.pre, 16) &&
                     (L.gemm2_permuted == nullptr ||
                      (unsigned long long)L.num_permuted * L.hidden * 2 < (1ull << 32));
  // a pending call whose outputs are this call's post, comb and pre is finished inside the
  // kernel: the fused kernel takes it when this call is deferred too and the pending
  // partial sums are a fused kernel's; the boundary kernel of the two-call form takes any
  bool defer_in = false;
  int st = MHC_OK;
  if (fused) {
    defer_in = h->pending && a->deferred && h->pend.ks_count > 0 && L.post == h->pend.post_out &&
               L.comb == h->pend.comb_out && L.pre == h->pend.pre_out && L.rows == h->pend.rows;
    st = defer_in ? MHC_OK : flush_pending(h, s);
  } else {
    st = take_pending(h, L, L.post, L.comb, L.pre, L.rows, s);
  }
  if (st != MHC_OK) return st;
  if (!fused) {
    st = launch_status(mhc::launch_boundary(L, s));
    if (st != MHC_OK) return st;
    return (a->deferred ? mhc_pre_coeffs_deferred : mhc_pre_coeffs)(
        h, L.residual_out, a->fn, a->scale, a->base, a->rms_eps, a->pre_eps, a->sinkhorn_eps,
        a->post_alpha, a->sinkhorn_iters, L.rows, a->pre_out, a->post_out, a->comb_out, s);
  }
  mhc::TileLaunch T;
  T.b = L;
  T.fn = a->fn;
  T.coef = mhc::CoeffEpilogue{};
  T.coef.scale = a->scale;
  T.coef.base = a->base;
  T.coef.K = h->hc_mult * h->hidden;
  T.coef.rms_eps = a->rms_eps;
  T.coef.pre_eps = a->pre_eps;
  T.coef.sk_eps = a->sinkhorn_eps;
  T.coef.alpha = a->post_alpha;
  T.coef.iters = a->sinkhorn_iters;
  T.next_pre = a->pre_out;
  T.next_post = a->post_out;
  T.next_comb = a->comb_out;
  T.part_out = nullptr;
  T.defer_in = defer_in;
  T.in_coef = defer_in ? mhc::pre_epilogue_args(h->pend) : mhc::CoeffEpilogue{};
  T.words = h->tile_words;
  T.tile_rows = h->tile_rows;
  T.wgs_per_xcd = h->tile_wgs_per_xcd;
  T.spread = h->tile_placement == MHC_TILE_SPREAD;
  if (!a->deferred) return launch_status(mhc::launch_boundary_tile(T, s));
  // deferred: the kernel leaves the next coefficients as partials; the call is pending
  // until a consumer or a flush finishes them
  float* part = h->tile_part[h->tile_part_next];  // not the pending call's
  T.part_out = part;
  h->pending = false;  // taken (defer_in) or flushed above
  st = launch_status(mhc::launch_boundary_tile(T, s));
  if (st != MHC_OK) return st;
  h->tile_part_next ^= 1;
  mhc::PreLaunch P = {};
  P.residual = L.residual_out;
  P.fn = a->fn;
  P.scale = a->scale;
  P.base = a->base;
  P.rms_eps = a->rms_eps;
  P.pre_eps = a->pre_eps;
  P.sinkhorn_eps = a->sinkhorn_eps;
  P.post_alpha = a->post_alpha;
  P.sinkhorn_iters = a->sinkhorn_iters;
  P.rows = L.rows;
  P.hidden = h->hidden;
  P.pre_out = a->pre_out;
  P.post_out = a->post_out;
  P.comb_out = a->comb_out;
  P.part = part;
  P.ks_count = mhc::boundary_tile_part_ks(h->hidden);
  h->pending = true;
  h->pend = P;
  return MHC_OK;
}

}  // namespace

int mhc_boundary_coeffs(mhc_handle h, const uint16_t* x_partials, int tp,
                        const uint16_t* residual, const float* post, const float* comb,
                        const float* pre, const uint16_t* norm_weight, float norm_eps, int rows,
                        uint16_t* residual_out, uint16_t* layer_input_out, uint8_t* mx_data_out,
                        uint8_t* mx_scale_out, const mhc_coeff_args* next, mhc_stream_t stream) {
  if (!h) return MHC_ERR_INVALID_ARG;
  if (rows < 0 || tp < 1) return MHC_ERR_SHAPE;
  if (rows > h->max_rows || tp > h->max_tp) return MHC_ERR_LIMIT;
  if (rows == 0) return MHC_OK;
  if (!x_partials || !pre) return MHC_ERR_INVALID_ARG;
  int st = check_mix(h, residual, post, comb, pre, norm_weight, norm_eps, residual_out,
                     layer_input_out, mx_data_out, mx_scale_out);
  if (st != MHC_OK) return st;
  if (!aligned(x_partials, 16)) return MHC_ERR_ALIGN;
  st = check_coeff_args(next);
  if (st != MHC_OK) return st;
  st = check_device(h);
  if (st != MHC_OK) return st;
  mhc::BoundaryLaunch L = {};
  L.x_partials = x_partials;
  L.tp = tp;
  fill_mix(h, L, residual, post, comb, pre, norm_weight, norm_eps, rows, residual_out,
           layer_input_out, mx_data_out, mx_scale_out);
  return boundary_then_coeffs(h, L, next, static_cast<hipStream_t>(stream));
}

int mhc_finalize_coeffs(mhc_handle h, const uint16_t* gemm2_permuted, int num_permuted,
                        const float* expert_weights, const int32_t* expanded_idx_to_permuted_idx,
                        const uint16_t* shared_output, const uint16_t* residual,
                        const float* post, const float* comb, const float* pre,
                        const uint16_t* norm_weight, float norm_eps, int rows,
                        uint16_t* residual_out, uint16_t* layer_input_out, uint8_t* mx_data_out,
                        uint8_t* mx_scale_out, const mhc_coeff_args* next, mhc_stream_t stream) {
  if (!h) return MHC_ERR_INVALID_ARG;
  if (rows < 0 || num_permuted < 1) return MHC_ERR_SHAPE;
  if (rows > h->max_rows) return MHC_ERR_LIMIT;
  if (rows == 0) return MHC_OK;
  if (!gemm2_permuted || !expert_weights || !expanded_idx_to_permuted_idx || !shared_output ||
      !pre)
    return MHC_ERR_INVALID_ARG;
  int st = check_mix(h, residual, post, comb, pre, norm_weight, norm_eps, residual_out,
                     layer_input_out, mx_data_out, mx_scale_out);
  if (st != MHC_OK) return st;
  if (!aligned(gemm2_permuted, 16) || !aligned(shared_output, 16) || !aligned(expert_weights, 4) ||
      !aligned(expanded_idx_to_permuted_idx, 4))
    return MHC_ERR_ALIGN;
  st = check_coeff_args(next);
  if (st != MHC_OK) return st;
  st = check_device(h);
  if (st != MHC_OK) return st;
  mhc::BoundaryLaunch L = {};
  L.gemm2_permuted = gemm2_permuted;
  L.num_permuted = num_permuted;
  L.expert_weights = expert_weights;
  L.idx = expanded_idx_to_permuted_idx;
  L.shared_output = shared_output;
  L.top_k = h->top_k;
  fill_mix(h, L, residual, post, comb, pre, norm_weight, norm_eps, rows, residual_out,
           layer_input_out, mx_data_out, mx_scale_out);
  return boundary_then_coeffs(h, L, next, static_cast<hipStream_t>(stream));
}

namespace {

int pre_coeffs_common(mhc_handle h, const uint16_t* residual, const uint16_t* fn,
                      const float* scale, const float* base, float rms_eps, float pre_eps,
                      float sinkhorn_eps, float post_alpha, int sinkhorn_iters, int rows,
                      float* pre_out, float* post_out, float* comb_out, mhc_stream_t stream,
                      bool deferred) {
  if (!h) return MHC_ERR_INVALID_ARG;
  if (rows < 0 || sinkhorn_iters < 0 || sinkhorn_iters > kMaxSinkhornIters) return MHC_ERR_SHAPE;
  if (!(rms_eps >= 0.0f) || !(sinkhorn_eps >= 0.0f)) return MHC_ERR_SHAPE;
  if (rows > h->max_rows) return MHC_ERR_LIMIT;
  if (rows == 0) return MHC_OK;
  if (!residual || !fn || !scale || !base || !pre_out || !post_out || !comb_out)
    return MHC_ERR_INVALID_ARG;
  if (!aligned(residual, 16) || !aligned(fn, 16) || !aligned(scale, 4) || !aligned(base, 4) ||
      !aligned(pre_out, 4) || !aligned(post_out, 4) || !aligned(comb_out, 4))
    return MHC_ERR_ALIGN;
  int st = check_device(h);
  if (st != MHC_OK) return st;
  mhc::PreLaunch L = {};
  L.residual = residual;
  L.fn = fn;
  L.scale = scale;
  L.base = base;
  L.rms_eps = rms_eps;
  L.pre_eps = pre_eps;
  L.sinkhorn_eps = sinkhorn_eps;
  L.post_alpha = post_alpha;
  L.sinkhorn_iters = sinkhorn_iters;
  L.rows = rows;
  L.hidden = h->hidden;
  L.pre_out = pre_out;
  L.post_out = post_out;
  L.comb_out = comb_out;
  L.part = h->pre_part;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  st = flush_pending(h, s);  // its partials are about to be overwritten
  if (st != MHC_OK) return st;
  if (!deferred) return launch_status(mhc::launch_pre_coeffs(L, s));
  st = launch_status(mhc::launch_pre_partial(L, s));
  if (st != MHC_OK) return st;
  h->pending = true;
  h->pend = L;
  return MHC_OK;
}

}  // namespace

int mhc_pre_coeffs(mhc_handle h, const uint16_t* residual, const uint16_t* fn,
                   const float* scale, const float* base, float rms_eps, float pre_eps,
                   float sinkhorn_eps, float post_alpha, int sinkhorn_iters, int rows,
                   float* pre_out, float* post_out, float* comb_out, mhc_stream_t stream) {
  return pre_coeffs_common(h, residual, fn, scale, base, rms_eps, pre_eps, sinkhorn_eps,
                           post_alpha, sinkhorn_iters, rows, pre_out, post_out, comb_out, stream,
                           false);
}

int mhc_pre_coeffs_deferred(mhc_handle h, const uint16_t* residual, const uint16_t* fn,
                            const float* scale, const float* base, float rms_eps, float pre_eps,
                            float sinkhorn_eps, float post_alpha, int sinkhorn_iters, int rows,
                            float* pre_out, float* post_out, float* comb_out,
                            mhc_stream_t stream) {
  return pre_coeffs_common(h, residual, fn, scale, base, rms_eps, pre_eps, sinkhorn_eps,
                           post_alpha, sinkhorn_iters, rows, pre_out, post_out, comb_out, stream,
                           true);
}

int mhc_pre_coeffs_flush(mhc_handle h, mhc_stream_t stream) {
  if (!h) return MHC_ERR_INVALID_ARG;
  if (!h->pending) return MHC_OK;
  int st = check_device(h);
  if (st != MHC_OK) return st;
  return flush_pending(h, static_cast<hipStream_t>(stream));
}

}  // extern "C"
