/*
 * mhc.h -- C ABI of the MI355X (gfx950) fused mHC boundary library, libmhc_amd.so.
 *
 * Pages cited (by title and section):
 *   boundary page   vllm.models.deepseek_v41.nvidia.specialized_decode.boundary.boundary
 *   all_reduce page vllm.models.deepseek_v41.nvidia.specialized_decode.boundary.all_reduce
 *   decode page     vllm.models.deepseek_v41.nvidia.specialized_decode.runtime.decode
 *
 * Conventions for every entry point
 *   - Tensor arguments are DEVICE pointers owned by the caller; the library
 *     never frees or keeps them. They must stay valid until the stream has
 *     passed the call.
 *   - bf16 tensors are passed as raw bit patterns (uint16_t), fp32 as float,
 *     E4M3 data and E8M0 scales as uint8_t. Every tensor is dense row-major in
 *     the shape given beside it. R = rows, n = hc_mult, H = hidden,
 *     T = tp, K = top_k.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL is the null
 *     stream), in stream order; nothing synchronizes the host.
 *   - Every call validates all of its arguments before any device work and
 *     returns an mhc_status. Nothing is launched when the status is not
 *     MHC_OK. Faults inside a launched kernel surface at the caller's next
 *     synchronization, as HIP reports them.
 *   - rows == 0 is a valid empty call: it returns MHC_OK and touches nothing
 *     (pointers are then not checked).
 *   - A handle owns a small device scratch area (per-row handoff words and
 *     epochs for the row RMS, an error word, coefficient partials). Calls on
 *     one handle must be serialized, i.e. issued on one stream or ordered by
 *     the caller; two overlapping calls on one handle race on its scratch.
 *   - The kernels that write a layer input (mhc_boundary and mhc_finalize with
 *     pre, mhc_first, mhc_collapse_norm) finish each row's RMS by a bounded
 *     wait between the workgroups of that row, which the library keeps
 *     co-resident (a launch uses at most half of the device's
 *     resident-workgroup capacity, in rounds if needed). A wait that
 *     exceeds the spin limit gives up and counts itself in the handle's error
 *     word (see mhc_get_errors); nothing hangs. The failure shows in the data:
 *     the part of the layer input whose wait gave up is NaN (bf16 NaN, E4M3
 *     NaN codes, E8M0 scale byte 0xFF), and so are the next coefficients of a
 *     fused call's row whose wait gave up. Such a row is marked in the handle
 *     (a late workgroup of the call that gave up may have left a handoff word
 *     that a later call would accept): every later call skips that row's
 *     waits and writes its wait-dependent outputs as NaN, until mhc_reset (or
 *     mhc_get_errors with clear) restores the handoff state. The new streams
 *     never depend on a wait and stay exact. A row's workgroups run on one XCD (ids
 *     congruent mod 8); where mhc_create finds the device dealing workgroup ids to its 8
 *     XCDs round-robin (it reads the hardware's XCC id over a probe grid), the handoff
 *     words go through that XCD's L2 (workgroup-scope stores, non-temporal polls that the
 *     CU's L1 does not keep), else through device-scope accesses
 *     (MHC_OPT_ROW_HANDOFF).
 *   - The only aliasing allowed is residual_out == residual (in-place update
 *     of the streams); any other overlap of inputs and outputs is undefined.
 *   - Alignment: bf16 tensors 16 bytes; fp32 and int32 tensors 4 bytes;
 *     mx_data_out 8 bytes. Otherwise MHC_ERR_ALIGN.
 */
#ifndef MHC_AMD_H
#define MHC_AMD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct mhc_ctx* mhc_handle; /* opaque */
typedef void* mhc_stream_t;         /* a hipStream_t */

enum mhc_status {
  MHC_OK = 0,
  MHC_ERR_INVALID_ARG = 1, /* null handle or required pointer, inconsistent optional outputs */
  MHC_ERR_SHAPE = 2,       /* a size that is negative, zero where it must be positive, or too large */
  MHC_ERR_ALIGN = 3,       /* a pointer not aligned as stated above */
  MHC_ERR_LIMIT = 4,       /* rows > max_rows or tp > max_tp of the handle */
  MHC_ERR_UNSUPPORTED = 5, /* hc_mult other than 4, or MXFP8 with hidden % 32 != 0 */
  MHC_ERR_HIP = 6,         /* a HIP runtime call failed (allocation, launch) */
  MHC_ERR_DEVICE = 7       /* the current HIP device is not the handle's device */
};

/* Human-readable name of a status code (a static string; never NULL). */
const char* mhc_status_string(int status);

/*
 * mhc_create -- a handle sized for every call it will serve.
 *
 * all_reduce page, BoundaryAllReduce.__init__: the fused kernel is sized once
 * by the model's hidden size, hc_mult, the largest row count it serves and
 * the MoE top_k, on one device. Here also by the largest number of TP
 * partial slices, max_tp.
 *   hidden   in [8, 65536], a multiple of 8 (16-byte vectors)  else MHC_ERR_SHAPE
 *   hc_mult  == 4                                         else MHC_ERR_UNSUPPORTED
 *   max_rows in [1, 65536], max_tp in [1, 64], top_k in [1, 64]  else MHC_ERR_SHAPE
 *   device   a valid HIP device index                     else MHC_ERR_HIP
 * Allocates the handle's device scratch on `device` (hipMalloc) and zeroes it
 * (synchronously) and picks the boundary block sizes: for calls of up to 32
 * rows 128, else 256, else 512 (the first whose row fits half an XCD's resident
 * workgroups and one polling wave; MHC_ERR_UNSUPPORTED if none does); for more
 * rows 256 when it fits (else the same size). On failure *out is set to NULL.
 * The sizes are checked before any HIP call.
 */
int mhc_create(int hidden, int hc_mult, int max_rows, int max_tp, int top_k, int device,
               mhc_handle* out);

/*
 * mhc_set_option -- knobs of a handle; none changes what is computed. The block size
 * and the elements per lane change the order in which a row's sum of squares is added
 * (the layer input may differ in the last bit of rare elements); a spin limit too small
 * to cover the row handoff makes it give up (see above); the scale layout chooses where
 * the MXFP8 scale bytes go. Takes effect for calls issued afterwards.
 *   MHC_OPT_BOUNDARY_BLOCK: threads per workgroup of the boundary kernels that write a
 *     layer input, 128, 256 or 512, for every call and row count (default: chosen
 *     per call from the row count, see mhc_create). Each thread owns 8 hidden
 *     elements of a row, so a row is split into ceil(H / (8 * block)) workgroups; a size
 *     giving more than 64 of them, or more than half an XCD's resident workgroups, is
 *     MHC_ERR_UNSUPPORTED. (The residual-only kernels use 512 threads, two elements
 *     each.)
 *     Other values: MHC_ERR_SHAPE.
 *   MHC_OPT_SPIN_LIMIT: polls (each followed by a short sleep) before a row-handoff
 *     wait gives up; >= 0, default 2^20. Negative: MHC_ERR_SHAPE.
 *   MHC_OPT_SCALE_LAYOUT: the layout of mx_scale_out in every call that writes an
 *     MXFP8 layer input (mhc_boundary, mhc_finalize, mhc_first, mhc_collapse_norm,
 *     mhc_boundary_coeffs, mhc_finalize_coeffs); the E4M3 data stays [R, H]:
 *       MHC_SCALE_ROW_MAJOR (default): [R, H/32], byte (r, b) at r * (H/32) + b.
 *       MHC_SCALE_SWIZZLED_128X4: the swizzled 128x4 layout the boundary page gives its
 *         MXFP8 layer input (empty_quantized_layer_input: FlashInfer's layout, the
 *         block-scale operand layout of block-scaled GEMMs). Rows are padded to a
 *         multiple of 128 and the H/32 blocks to a multiple of 4; with KT = padded
 *         blocks / 4, byte (r, b) is at
 *           ((r / 128) * KT + b / 4) * 512 + (r % 32) * 16 + ((r / 32) % 4) * 4 + b % 4,
 *         i.e. one 512-byte tile per 128 rows x 4 blocks, tiles row-major. The buffer
 *         holds mhc_mxfp8_scale_bytes(R, H, MHC_SCALE_SWIZZLED_128X4) bytes; the
 *         padding bytes (rows >= R, blocks >= H/32) are not written.
 *     Other values: MHC_ERR_SHAPE.
 *   MHC_OPT_LANE_ELEMS: the fewest hidden elements per thread that the kernels writing a
 *     layer input (mhc_boundary, mhc_finalize, mhc_collapse_norm and the fused calls'
 *     fallback) may use: 2 (default), 4 or 8. With e elements per thread (8: 16-byte
 *     vectors, 4: 8-byte, 2: 4-byte) a workgroup has 8 / e times the threads of the
 *     eight-per-thread size, so a row keeps the same number of workgroups. A call takes the
 *     fewest e >= the option whose workgroup exists (at most 512 threads) and fits the
 *     co-residency limit, if the block size is chosen per call, the call has at most 128
 *     rows and it then needs no more rounds than at 8; otherwise 8. The new streams are
 *     identical for every e (every element's arithmetic is the same). Other values:
 *     MHC_ERR_SHAPE.
 *   MHC_OPT_TILE_PLACEMENT: where the fused calls' single kernel (mhc_boundary_coeffs,
 *     mhc_finalize_coeffs) runs the 256-element chunks of a 16-row tile:
 *       MHC_TILE_SPREAD (default): chunk c of every tile on XCD c % 8, so each XCD reads
 *         only its chunks' rows of fn, and a call of few rows still uses every XCD;
 *       MHC_TILE_PER_XCD: all chunks of a tile on one XCD (tiles dealt to XCDs), ahead
 *         when the same fn is reused by consecutive calls while it is still cached.
 *     Results are identical either way (the same arithmetic per chunk and the same order
 *     of every sum). Other values: MHC_ERR_SHAPE.
 *   MHC_OPT_ROW_HANDOFF: how the workgroups of a row exchange their partial sums in
 *     the layer-input kernels (mhc_boundary, mhc_finalize, mhc_first, mhc_collapse_norm and
 *     the fused calls' fallback):
 *       MHC_HANDOFF_XCD (default where available): through the L2 of the row's XCD;
 *         MHC_ERR_UNSUPPORTED on a device that mhc_create did not find dealing workgroup
 *         ids to its XCDs round-robin;
 *       MHC_HANDOFF_DEVICE (default otherwise): device-scope stores and polls.
 *     Results are identical either way. Other values: MHC_ERR_SHAPE.
 * Unknown options: MHC_ERR_INVALID_ARG.
 */
enum mhc_option {
  MHC_OPT_BOUNDARY_BLOCK = 1,
  MHC_OPT_SPIN_LIMIT = 2,
  MHC_OPT_SCALE_LAYOUT = 3,
  MHC_OPT_LANE_ELEMS = 4,
  MHC_OPT_TILE_PLACEMENT = 5,
  MHC_OPT_ROW_HANDOFF = 6
};
enum mhc_scale_layout { MHC_SCALE_ROW_MAJOR = 0, MHC_SCALE_SWIZZLED_128X4 = 1 };
enum mhc_tile_placement { MHC_TILE_PER_XCD = 0, MHC_TILE_SPREAD = 1 };
enum mhc_row_handoff { MHC_HANDOFF_DEVICE = 0, MHC_HANDOFF_XCD = 1 };
int mhc_set_option(mhc_handle h, int option, int value);

/*
 * mhc_mxfp8_scale_bytes -- the size in bytes of mx_scale_out for `rows` rows of `hidden`
 * elements in a scale layout (see MHC_OPT_SCALE_LAYOUT): rows * hidden/32 row-major,
 * roundup(rows, 128) * roundup(hidden/32, 4) swizzled. Host only (no device work).
 * boundary page, empty_quantized_layer_input: the scale buffer of an MXFP8 layer input
 * is sized from the token count and hidden size.
 *   rows >= 0, hidden > 0 and a multiple of 32  else MHC_ERR_SHAPE
 *   layout a mhc_scale_layout                   else MHC_ERR_SHAPE
 *   bytes  a host pointer                       else MHC_ERR_INVALID_ARG
 */
int mhc_mxfp8_scale_bytes(int rows, int hidden, int layout, uint64_t* bytes);

/*
 * mhc_get_errors -- the number of row-handoff waits that gave up since the
 * handle was created or last cleared. Enqueues a device-to-host copy of the
 * error word on `stream` and waits for that stream (so it follows every call
 * issued before it on `stream`); with clear != 0, then re-zeroes the whole
 * handoff state on `stream` as mhc_reset does (the error word alone is not
 * enough: a count above zero means stale handoff words may be left behind).
 * count must be a host pointer.
 */
int mhc_get_errors(mhc_handle h, unsigned* count, int clear, mhc_stream_t stream);

/* Frees the handle and its scratch (synchronizes the device first). NULL is a no-op. */
int mhc_destroy(mhc_handle h);

/*
 * mhc_reset -- re-zero the handle's handoff words, epochs and error word on
 * `stream` (a fill kernel, so it may be captured in a graph).
 *
 * all_reduce page, BoundaryAllReduce.reset: drop what an aborted step left
 * behind. Completed calls leave the handoff state consistent by themselves;
 * this is only needed after a call whose kernels did not complete or whose
 * waits gave up, and then it is required: until it runs, every call writes
 * its wait-dependent outputs as NaN (see the conventions above).
 */
int mhc_reset(mhc_handle h, mhc_stream_t stream);

/*
 * mhc_boundary -- the fused boundary on TP-partial slices.
 *
 * boundary page, module docstring and Boundaries._reduce; all_reduce page,
 * BoundaryAllReduce.__call__. For each row r and hidden index h:
 *   x[r,h]      = bf16( sum_t x_partials[t,r,h] )                (t ascending, fp32)
 *   s'[r,i,h]   = bf16( sum_j comb[r,i,j] * residual[r,j,h] + post[r,i] * x[r,h] )
 *   y[r,h]      = sum_j pre[r,j] * s'[r,j,h]
 *   layer[r,h]  = bf16( y[r,h] * (mean_h y[r,:]^2 + norm_eps)^(-1/2) * norm_weight[h] )
 * and optionally the MXFP8 form of layer[]: per block of 32 contiguous
 * elements of a row, e = the smallest integer with max|block| <= 448 * 2^e
 * (-127 for an all-zero block, clamped to [-127,127]); scale byte = e + 127;
 * data = E4M3 (OCP, FN variant) of layer * 2^-e, nearest-even.
 *
 *   x_partials      [T, R, H] bf16, T = tp in [1, max_tp]
 *   residual        [R, n, H] bf16 (the hc residual streams)
 *   post            [R, n] fp32;  comb [R, n, n] fp32 (i = output stream, j = input stream)
 *   pre             [R, n] fp32, or NULL for residual-only (then norm_weight and
 *                   layer_input_out must be NULL and no MXFP8 may be asked for)
 *   norm_weight     [H] bf16;  norm_eps >= 0
 *   residual_out    [R, n, H] bf16, may equal residual
 *   layer_input_out [R, H] bf16
 *   mx_data_out     [R, H] E4M3 bytes and mx_scale_out [R, H/32] E8M0 bytes (or the
 *                   swizzled layout, see MHC_OPT_SCALE_LAYOUT), both NULL (no MXFP8)
 *                   or both set (needs pre and H % 32 == 0)
 */
int mhc_boundary(mhc_handle h, const uint16_t* x_partials, int tp, const uint16_t* residual,
                 const float* post, const float* comb, const float* pre,
                 const uint16_t* norm_weight, float norm_eps, int rows, uint16_t* residual_out,
                 uint16_t* layer_input_out, uint8_t* mx_data_out, uint8_t* mx_scale_out,
                 mhc_stream_t stream);

/*
 * mhc_boundary_noalloc -- mhc_boundary for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, hosts that forbid hipMalloc): no
 * handle, and no allocation by the library at any call.
 *
 * Computes exactly what mhc_boundary computes on a handle with default options (same
 * kernels, launch shape and order of sums, so the outputs are bit-identical), with the
 * same arguments, layouts, aliasing and validation, hc_mult = 4, on the current HIP device.
 * (The row handoff uses device-scope accesses, MHC_HANDOFF_DEVICE: the outputs are the same.)
 * The row handoff's words, epochs and marks live in a fixed array of 1152.25 KiB in device
 * memory (one copy per GPU, held until the process ends) instead of a handle's scratch:
 *   rows   in [0, 1024]   (0: no-op)          else MHC_ERR_LIMIT (beyond the array)
 *   hidden a multiple of 8, at most 16384     else MHC_ERR_SHAPE / MHC_ERR_LIMIT
 *   tp     in [1, 64]                         else MHC_ERR_SHAPE / MHC_ERR_LIMIT
 * The first call on each device sets it up: it looks up the array's address on that device
 * and the kernels' occupancy there, and zeroes the array on `stream` (a fill kernel, ahead
 * of the call's own). Make one call outside any graph capture first. reset != 0 zeroes the
 * array again on `stream` before the call: needed only after a call whose handoff wait
 * gave up (its NaN outputs show it; the conventions above apply, with this array for the
 * handle's scratch, and no count is kept).
 * Every call on a device shares that device's array, which keeps the last call's state:
 * calls that overlap on one device (different streams, or different host threads without
 * ordering) race on it and give wrong layer inputs. Issue them in one stream order.
 */
int mhc_boundary_noalloc(int hidden, const uint16_t* x_partials, int tp,
                         const uint16_t* residual, const float* post, const float* comb,
                         const float* pre, const uint16_t* norm_weight, float norm_eps, int rows,
                         uint16_t* residual_out, uint16_t* layer_input_out, uint8_t* mx_data_out,
                         uint8_t* mx_scale_out, int reset, mhc_stream_t stream);

/*
 * mhc_residual_only -- reduce and mix only: writes residual_out and nothing else.
 *
 * boundary page, Boundaries.post_only and Boundaries._reduce (without a pre
 * the kernel writes only the streams: before an Engram injection and for the
 * final collapse). Same as mhc_boundary with pre = NULL.
 */
int mhc_residual_only(mhc_handle h, const uint16_t* x_partials, int tp, const uint16_t* residual,
                      const float* post, const float* comb, int rows, uint16_t* residual_out,
                      mhc_stream_t stream);

/*
 * mhc_finalize -- the fused boundary on an unfinalized MoE output.
 *
 * boundary page, Boundaries._reduce (MoE branch); all_reduce page,
 * BoundaryAllReduce.finalize. Identical to mhc_boundary except that
 *   x[r,h] = bf16( shared_output[r,h] + sum_k expert_weights[r,k] *
 *                  gemm2_permuted[ expanded_idx_to_permuted_idx[r*K + k], h ] )
 * (k ascending, fp32), with K the handle's top_k.
 *   gemm2_permuted               [num_permuted, H] bf16, num_permuted >= 1
 *   expert_weights               [R, K] fp32
 *   expanded_idx_to_permuted_idx [R*K] int32; an entry outside [0, num_permuted)
 *                                contributes nothing (it is never dereferenced)
 *   shared_output                [R, H] bf16 (required)
 * pre == NULL gives the residual-only form, as for mhc_boundary.
 */
int mhc_finalize(mhc_handle h, const uint16_t* gemm2_permuted, int num_permuted,
                 const float* expert_weights, const int32_t* expanded_idx_to_permuted_idx,
                 const uint16_t* shared_output, const uint16_t* residual, const float* post,
                 const float* comb, const float* pre, const uint16_t* norm_weight, float norm_eps,
                 int rows, uint16_t* residual_out, uint16_t* layer_input_out,
                 uint8_t* mx_data_out, uint8_t* mx_scale_out, mhc_stream_t stream);

/*
 * mhc_collapse_mean -- out[r,h] = bf16( (1/n) * sum_i streams[r,i,h] ).
 *
 * boundary page, Boundaries.sublayer (the aux output is the mean of the
 * streams over the stream axis); decode page, SpecializedDecode.run (the
 * same mean after the final residual-only reduction).
 *   streams [R, n, H] bf16 -> out [R, H] bf16
 */
int mhc_collapse_mean(mhc_handle h, const uint16_t* streams, int rows, uint16_t* out,
                      mhc_stream_t stream);

/*
 * mhc_first -- the first layer's entry: hc copies of the embedding as the
 * streams, and the first sublayer's input.
 *
 * boundary page, Boundaries.first: every residual stream starts as a copy of
 * the embedding x, and the first pre-mix is the identity on stream 0, so the
 * layer input is x normalized with the sublayer's norm:
 *   residual_out[r, i, :] = x[r, :]                     (bit for bit, every i)
 *   layer[r, h] = bf16( x[r,h] * (mean_h x[r]^2 + eps)^(-1/2) * w[h] )
 * and the optional MXFP8 form as for mhc_boundary. The coefficients of the
 * first sublayer come from mhc_pre_coeffs on residual_out.
 *   x [R, H] bf16;  norm_weight [H] bf16;  eps >= 0
 *   residual_out [R, n, H] bf16 (must not overlap x);  layer_input_out [R, H] bf16
 *   mx_data_out, mx_scale_out: both NULL or both set (hidden % 32 == 0)
 */
int mhc_first(mhc_handle h, const uint16_t* x, const uint16_t* norm_weight, float eps, int rows,
              uint16_t* residual_out, uint16_t* layer_input_out, uint8_t* mx_data_out,
              uint8_t* mx_scale_out, mhc_stream_t stream);

/*
 * mhc_collapse_norm -- the head after the layers: the streams collapsed with
 * the last pre-mix, then the final norm.
 *
 * decode page, _head (after Boundaries.post_only): the collapse is its own op
 * there, so it is rounded to bf16 once before the norm:
 *   y[r, h]   = bf16( sum_j pre[r, j] * s[r, j, h] )
 *   out[r, h] = bf16( y * (mean_h y^2 + eps)^(-1/2) * w[h] )
 * and the optional MXFP8 form as for mhc_boundary.
 *   residual [R, n, H] bf16 (read only);  pre [R, n] fp32;  norm_weight [H] bf16
 *   out [R, H] bf16;  mx_data_out, mx_scale_out: both NULL or both set
 */
int mhc_collapse_norm(mhc_handle h, const uint16_t* residual, const float* pre,
                      const uint16_t* norm_weight, float eps, int rows, uint16_t* out,
                      uint8_t* mx_data_out, uint8_t* mx_scale_out, mhc_stream_t stream);

/*
 * mhc_pre_coeffs -- the next sublayer's mHC coefficients from the streams.
 *
 * boundary page, Boundaries.sublayer and Boundaries._pre: the coefficient
 * call takes the streams, fn, scale, base, rms_norm_eps, hc_eps (as the pre
 * eps and again as the Sinkhorn eps), hc_post_alpha and hc_sinkhorn_iters.
 * With v = residual[r] flattened stream-major (k = i*H + h), NC = 2n + n*n:
 *   inv     = (mean_k v[k]^2 + rms_eps)^(-1/2)
 *   l[c]    = inv * sum_k v[k] * fn[k, c]                     (c < NC)
 *   l'[c]   = l[c] * scale[g(c)] + base[c],  g = 0 for c < n, 1 for c < 2n, else 2
 *   pre[i]  = sigmoid(l'[i]) + pre_eps
 *   post[i] = post_alpha * sigmoid(l'[n + i])
 *   comb    = A after sinkhorn_iters rounds of {A <- A / (rowsum + sinkhorn_eps);
 *             A <- A / (colsum + sinkhorn_eps)}, starting from
 *             A[i,j] = exp(l'[2n+n*i+j] - max_j l'[2n+n*i+j])
 *   residual [R, n, H] bf16;  fn [n*H, NC] bf16 row-major (16-byte aligned)
 *   scale [3] fp32;  base [NC] fp32;  sinkhorn_iters in [0, 1000]
 *   pre_out [R, n], post_out [R, n], comb_out [R, n, n], fp32
 */
int mhc_pre_coeffs(mhc_handle h, const uint16_t* residual, const uint16_t* fn,
                   const float* scale, const float* base, float rms_eps, float pre_eps,
                   float sinkhorn_eps, float post_alpha, int sinkhorn_iters, int rows,
                   float* pre_out, float* post_out, float* comb_out, mhc_stream_t stream);

/*
 * mhc_pre_coeffs_deferred -- mhc_pre_coeffs (same arguments, same results, bit for bit)
 * with its last step left to the call that consumes it.
 *
 * Runs the split-K projection now and records the call as pending on the handle. The
 * next mhc_boundary, mhc_finalize or mhc_residual_only on the handle whose post and
 * comb are this call's post_out and comb_out (and whose pre, if any, is pre_out), with
 * the same rows, finishes the coefficients inside its own kernel (while its loads are
 * in flight) and writes pre_out, post_out and comb_out as well. Any other call on the
 * handle, a mhc_pre_coeffs or mhc_pre_coeffs_deferred call included, first enqueues the
 * pending epilogue as mhc_pre_coeffs would have. Until then the outputs are not
 * written: a caller that reads them otherwise calls mhc_pre_coeffs_flush first.
 * scale, base and the three outputs are used when that later call runs, so they must
 * stay allocated until it has (the streams and fn only until this call has run).
 * mhc_destroy drops a pending call unwritten.
 * Errors: as mhc_pre_coeffs (a failing call records nothing).
 */
int mhc_pre_coeffs_deferred(mhc_handle h, const uint16_t* residual, const uint16_t* fn,
                            const float* scale, const float* base, float rms_eps, float pre_eps,
                            float sinkhorn_eps, float post_alpha, int sinkhorn_iters, int rows,
                            float* pre_out, float* post_out, float* comb_out,
                            mhc_stream_t stream);

/*
 * mhc_pre_coeffs_flush -- enqueue the epilogue of a pending deferred coefficient call on
 * `stream` (nothing if none is pending), after which its outputs are complete in stream
 * order. MHC_ERR_INVALID_ARG for a NULL handle.
 */
int mhc_pre_coeffs_flush(mhc_handle h, mhc_stream_t stream);

/*
 * The arguments of a coefficient call (as mhc_pre_coeffs) carried by the fused calls
 * below. A host struct, read during the call only; the pointers are device pointers
 * with mhc_pre_coeffs's layouts and alignments. deferred = 1 makes the coefficient call
 * a deferred one (as mhc_pre_coeffs_deferred): the fused kernel leaves the coefficients
 * as partial sums in the handle and the call stays pending; its outputs are written by
 * the next call that consumes them (a boundary, finalize, residual-only or fused call
 * whose post and comb, and pre if it takes one, are these outputs, for the same rows),
 * by the epilogue that any other call enqueues first, or by mhc_pre_coeffs_flush. Other
 * values than 0 and 1 give MHC_ERR_INVALID_ARG.
 */
typedef struct mhc_coeff_args {
  const uint16_t* fn;       /* [n*H, 2n + n*n] bf16 row-major, 16-byte aligned */
  const float* scale;       /* [3] */
  const float* base;        /* [2n + n*n] */
  float rms_eps, pre_eps, sinkhorn_eps, post_alpha;
  int sinkhorn_iters;       /* [0, 1000] */
  int deferred;             /* 0 or 1: leave the coefficients pending (see below) */
  float* pre_out;           /* [R, n] */
  float* post_out;          /* [R, n] */
  float* comb_out;          /* [R, n, n] */
} mhc_coeff_args;

/*
 * mhc_boundary_coeffs -- mhc_boundary followed by mhc_pre_coeffs on its new streams, in
 * one kernel.
 *
 * boundary page, Boundaries.sublayer: a sublayer's boundary returns the new streams and
 * the next sublayer's input, and the next coefficient call (Boundaries._pre) runs on
 * those streams. This call computes exactly what
 *   mhc_boundary(h, x_partials, tp, residual, post, comb, pre, norm_weight, norm_eps,
 *                rows, residual_out, layer_input_out, mx_data_out, mx_scale_out, s);
 *   mhc_pre_coeffs(h, residual_out, next->fn, next->scale, next->base, next->rms_eps,
 *                  next->pre_eps, next->sinkhorn_eps, next->post_alpha,
 *                  next->sinkhorn_iters, rows, next->pre_out, next->post_out,
 *                  next->comb_out, s);
 * compute, but the projection is taken from the new streams while they are in
 * registers (no second read of the streams, no separate launches). The new streams are
 * bit-identical to mhc_boundary's; the layer input, its MXFP8 form and the coefficients
 * differ from the two calls' by the order of their sums only (the row sums are split
 * into 256-element pieces). A layer input is required (pre, norm_weight and
 * layer_input_out non-NULL). Arguments, layouts, aliasing and errors as the two calls,
 * plus MHC_ERR_INVALID_ARG for a NULL `next`; next's outputs must not overlap any other
 * argument. The single kernel runs when rows <= min(max_rows, 1024), post, comb and pre
 * are 16-byte aligned, a row's 256-element pieces fit the workgroups one XCD holds at
 * once (H <= 8192 on MI355X) and, for mhc_finalize_coeffs, the permuted expert rows span
 * less than 4 GiB (num_permuted * hidden * 2 bytes); otherwise the call runs the two calls
 * (same results as above). A pending deferred coefficient call whose outputs are this call's post, comb and
 * pre (same rows) is finished inside the kernel when this call is deferred too and the
 * pending call was a fused one (its partial sums are the fused kernel's); in the two-call
 * form the boundary kernel finishes it; otherwise its epilogue is enqueued first.
 * Concurrency: the single kernel may occupy every resident slot of an XCD for its tile's
 * workgroups, which wait on one another. Kernels of other streams only delay it, but two
 * of these calls running at the same time on different streams can each hold part of an
 * XCD and wait for the rest: their waits then end at the spin limit (counted by
 * mhc_get_errors) with NaN outputs. Issue fused calls of one device on one stream.
 */
int mhc_boundary_coeffs(mhc_handle h, const uint16_t* x_partials, int tp,
                        const uint16_t* residual, const float* post, const float* comb,
                        const float* pre, const uint16_t* norm_weight, float norm_eps, int rows,
                        uint16_t* residual_out, uint16_t* layer_input_out, uint8_t* mx_data_out,
                        uint8_t* mx_scale_out, const mhc_coeff_args* next, mhc_stream_t stream);

/*
 * mhc_finalize_coeffs -- mhc_finalize followed by mhc_pre_coeffs on its new streams, in
 * one kernel: as mhc_boundary_coeffs with mhc_finalize's sublayer-output arguments
 * (all_reduce page, BoundaryAllReduce finalize; boundary page, Boundaries.sublayer).
 */
int mhc_finalize_coeffs(mhc_handle h, const uint16_t* gemm2_permuted, int num_permuted,
                        const float* expert_weights, const int32_t* expanded_idx_to_permuted_idx,
                        const uint16_t* shared_output, const uint16_t* residual,
                        const float* post, const float* comb, const float* pre,
                        const uint16_t* norm_weight, float norm_eps, int rows,
                        uint16_t* residual_out, uint16_t* layer_input_out, uint8_t* mx_data_out,
                        uint8_t* mx_scale_out, const mhc_coeff_args* next, mhc_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MHC_AMD_H */
