/*
 * nvfp4.h -- C ABI of libnvfp4.so: NVFP4 two-level block quantization of 2-D
 * bf16 tensors on an AMD Instinct MI355X (gfx950).
 *
 * The method (what each call computes) is the one described by
 *   - the VideoX-Fun page "videox_fun/utils/fp4_optimization.py": module
 *     constants, quantize_weight_to_float4, dequantize_weight_from_float4,
 *     _float4_round;
 *   - the verl tutorial page "linear.py -- QATLinear": section 1 (FP4
 *     fake-quant kernel), 2 (straight-through estimator), 4 (fused-sibling
 *     weight amax), 5 (activation observer).
 *
 * Numerics, fixed for every call (all arithmetic IEEE binary32, no FMA
 * contraction, subnormals kept):
 *   amax   = max |x|                                   (raw, no clamp)
 *   gs     = 2688 / max(amax, 1e-12f)                   2688 = 448 * 6
 *   per 16-element block of one row:
 *     S    = E4M3_RNE_SATURATE((block_amax / 6) * gs)   one byte
 *     sd   = decode(S) / gs ;  sq = max(sd, 1e-12f)
 *     q    = x / sq ;  idx = E2M1 round-to-nearest-even of min(|q|, 6)
 *            onto {0, .5, 1, 1.5, 2, 3, 4, 6}
 *     code = idx | 8 * (q < 0)                         4 bits
 *   fake-quant / unpack output = bf16_RNE(LUT[code] * sd), LUT[8..15] = -LUT[0..7]
 *
 * Conventions shared by every call:
 *   - Tensor pointers are DEVICE pointers; tensors are row-major and
 *     contiguous (row stride = cols).  bf16 travels as 16-bit patterns.
 *   - The caller owns all memory.  The library allocates nothing and keeps no
 *     mutable state between calls; calls on different streams may run
 *     concurrently as long as their buffers do not overlap.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *     enqueues work on it and never synchronises the host; results are ready
 *     when the stream reaches them.
 *   - Arguments are checked on the host before anything is enqueued; a failed
 *     check returns an error code and enqueues nothing.  A kernel that fails to
 *     launch returns NVFP4_ERR_HIP.  Asynchronous device faults surface at the
 *     caller's next synchronisation.
 *   - Inputs must be finite; NaN and Inf inputs give unspecified bytes.
 *   - Shapes: rows >= 0 and cols >= 1; rows == 0 is a valid empty tensor.
 *     Blocks are 16 consecutive columns of one row and never straddle rows.  A
 *     row whose length is not a multiple of 16 is zero-padded to
 *     nbr = ceil(cols / 16) blocks (VideoX-Fun page, quantize_weight_to_float4):
 *     the pad never changes a block max, the packed codes and scales keep the
 *     padded layout, and bf16 outputs have exactly cols columns.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum nvfp4_status {
    NVFP4_OK = 0,
    NVFP4_ERR_NULL = 1,     /* a required pointer is NULL                          */
    NVFP4_ERR_SHAPE = 2,    /* rows < 0, cols < 1, or a size that overflows        */
    NVFP4_ERR_ALIGN = 3,    /* a pointer is not aligned as the call requires       */
    NVFP4_ERR_OVERLAP = 4,  /* an output overlaps an input or another output       */
    NVFP4_ERR_ARG = 5,      /* a bad mode, decay, or group count                   */
    NVFP4_ERR_HIP = 6       /* the HIP runtime refused a launch                    */
} nvfp4_status;

enum {
    NVFP4_OBS_STATIC_MINMAX = 0,  /* running maximum of the observed amax          */
    NVFP4_OBS_EMA = 1             /* exponential moving average of the amax        */
};

/* Largest number of tensors one nvfp4_amax launch covers; longer lists are
 * split into several launches on the same stream. */
#define NVFP4_AMAX_GROUP_MAX 8

/*
 * nvfp4_amax -- per-tensor |x| maximum, or the shared maximum of fused
 * siblings (verl QATLinear page, section 4: the max over every sibling's
 * weight.abs().max(); VideoX-Fun page, quantize_weight_to_float4: the
 * tensor-wide abs().amax()).
 *
 *   xs[i]      device pointer to numels[i] bf16 values (any shape, contiguous),
 *              16-byte aligned; may be NULL when numels[i] == 0
 *   numels[i]  element count of tensor i, >= 0
 *   n          number of tensors, >= 1 (xs and numels are HOST arrays of n)
 *   amax       device fp32 scalar, 4-byte aligned.  accumulate == 0:
 *              *amax := max over the group (+0.0 for an all-empty group);
 *              accumulate != 0: *amax := max(*amax, max over the group), where
 *              a negative prior value (such as -1) counts as "none".
 * Errors: NULL (xs, numels, amax, or xs[i] with numels[i] > 0), SHAPE
 * (numels[i] < 0), ARG (n < 1), ALIGN, HIP.
 */
nvfp4_status nvfp4_amax(const void* const* xs, const int64_t* numels, int n,
                        float* amax, int accumulate, void* stream);

/*
 * nvfp4_fake_quant -- bf16 [rows, cols] -> bf16 [rows, cols] fake-quantized
 * values: quantize then dequantize (verl QATLinear page, section 1, the
 * rescaled grid value; VideoX-Fun page, the divide-by-gs scale convention).
 * Its straight-through backward (section 2) is the identity and has no call.
 *
 *   x, y       device bf16, 16-byte aligned.  y == x (exact in-place) is allowed;
 *              any other overlap is an error.
 *   amax_in    NULL: the amax is computed from x first and written to amax_out
 *              (required then).  Non-NULL: device fp32 amax to use as is (a
 *              shared sibling amax or an observer state); x is read once.
 *   amax_out   device fp32, written only when amax_in is NULL; may be NULL otherwise.
 */
nvfp4_status nvfp4_fake_quant(const void* x, void* y, int64_t rows, int64_t cols,
                              const float* amax_in, float* amax_out, void* stream);

/*
 * nvfp4_fake_quant_group -- fake-quantize n tensors that share one amax, the
 * fused siblings of one layer (verl QATLinear page, section 4: q, k and v, or
 * gate and up, are fake-quantized with the maximum over all of them).  Each
 * output equals nvfp4_fake_quant of its tensor with that shared amax; tensors
 * whose rows are whole blocks are fake-quantized together, one launch per
 * NVFP4_AMAX_GROUP_MAX of them (ragged tensors get a launch each).
 *
 *   xs, ys       HOST arrays of n device pointers: bf16 [rows[i], cols[i]],
 *                16-byte aligned; NULL allowed for an empty tensor.  ys[i] ==
 *                xs[i] (exact in-place) is allowed; any other overlap between
 *                an output and an input or another output is an error.
 *   rows, cols   HOST arrays of n shapes, each as for nvfp4_fake_quant
 *   n            >= 1
 *   amax_in      NULL: the amax of the whole group is computed first (one
 *                grouped pass, as nvfp4_amax) into amax_out (required then).
 *                Non-NULL: device fp32 amax used for every tensor.
 *   amax_out     as for nvfp4_fake_quant
 * Errors: NULL, SHAPE, ALIGN, OVERLAP, ARG (n < 1), HIP.
 */
nvfp4_status nvfp4_fake_quant_group(const void* const* xs, void* const* ys, const int64_t* rows,
                                    const int64_t* cols, int n, const float* amax_in,
                                    float* amax_out, void* stream);

/*
 * nvfp4_fake_quant_dual -- one bf16 [rows, cols] tensor fake-quantized under
 * two amaxes, reading x once: the activation of a layer fake-quantized with
 * the states of two observers (verl QATLinear page, section 5; for instance
 * static running max and EMA side by side).  y0 equals nvfp4_fake_quant(x,
 * amax_in = amax0) and y1 the same with amax1.  The stream traffic is 6 bytes
 * per element instead of 8 for two calls.
 *
 *   x            device bf16 [rows, cols], 16-byte aligned
 *   amax0, amax1 device fp32 amaxes (required), 4-byte aligned
 *   y0, y1       device bf16 [rows, cols], 16-byte aligned; either one (not
 *                both) may be x itself; y0 and y1 must not overlap each other,
 *                the amaxes, or x otherwise
 * Errors: NULL, SHAPE, ALIGN, OVERLAP, HIP.
 */
nvfp4_status nvfp4_fake_quant_dual(const void* x, int64_t rows, int64_t cols, const float* amax0,
                                   void* y0, const float* amax1, void* y1, void* stream);

/*
 * nvfp4_quantize_pack -- bf16 [rows, cols] -> packed NVFP4 (VideoX-Fun page,
 * quantize_weight_to_float4, returning nibbles, E4M3 block scales and the
 * fp32 per-tensor factor).
 *
 *   x             device bf16 [rows, cols], 16-byte aligned
 *   amax_in/out   as for nvfp4_fake_quant
 *   packed        device uint8 [rows, 8 * nbr], 8-byte aligned; byte i of a row
 *                 holds the code of (padded) column 2i in its low nibble and of
 *                 column 2i+1 in its high nibble; padding columns get code 0
 *   scales        device uint8 [rows, nbr], E4M3 (float8_e4m3fn) bytes,
 *                 row-major, one per block
 *   global_scale  device fp32: gs (not the amax), 4-byte aligned
 * Outputs must not overlap x, amax_in or each other.
 */
nvfp4_status nvfp4_quantize_pack(const void* x, int64_t rows, int64_t cols,
                                 const float* amax_in, float* amax_out,
                                 uint8_t* packed, uint8_t* scales, float* global_scale,
                                 void* stream);

/*
 * nvfp4_dequant_unpack -- packed NVFP4 -> bf16 [rows, cols] (VideoX-Fun page,
 * dequantize_weight_from_float4: nibble -> E2M1 value, times
 * decode(scale) / gs, rounded to bf16).  Layouts as nvfp4_quantize_pack writes
 * them; scale bytes outside 0x00..0x7E (never written by the pack) give
 * unspecified outputs.  packed 8-byte aligned, y 16-byte aligned; y must not
 * overlap the inputs.
 */
nvfp4_status nvfp4_dequant_unpack(const uint8_t* packed, const uint8_t* scales,
                                  const float* global_scale, int64_t rows, int64_t cols,
                                  void* y, void* stream);

/*
 * nvfp4_linear -- y = x . w^T + b for a weight w stored as packed NVFP4: the
 * layer's linear run on the dequantized weight (VideoX-Fun page, the
 * per-forward reconstruction, where the packed weight is dequantized to bf16
 * before the module's own forward).  w is exactly the bf16 tensor that
 * nvfp4_dequant_unpack writes, but it is decoded in registers and never stored.
 * Products and sums are binary32 (the weight and x are bf16, so every product is
 * exact); the order of the sums is fixed by the kernel for a shape and device
 * (it may depend on the device's CU count) and does not change from run to run;
 * y is rounded to bf16 (nearest even) once, after the bias is added.
 *
 *   x             device bf16 [m, k], 16-byte aligned
 *   packed        device uint8 [n, k / 2], the codes of w as nvfp4_quantize_pack
 *                 writes them, 16-byte aligned
 *   scales        device uint8 [n, k / 16], E4M3 block scales, 2-byte aligned
 *   global_scale  device fp32 gs of w
 *   bias          device bf16 [n], 2-byte aligned, or NULL for none
 *   y             device bf16 [m, n], 2-byte aligned; must not overlap an input
 *   m >= 0, n >= 0; k >= 32 and k % 32 == 0 (other widths: unpack, then a GEMM)
 * Errors: SHAPE, NULL, ALIGN, OVERLAP, HIP.
 */
nvfp4_status nvfp4_linear(const void* x, int64_t m, int64_t k, const uint8_t* packed,
                          const uint8_t* scales, const float* global_scale, int64_t n, const void* bias,
                          void* y, void* stream);

/*
 * nvfp4_observer_update -- one activation-observer step on device scalars
 * (verl QATLinear page, section 5):
 *   NVFP4_OBS_STATIC_MINMAX:  *state := max(*state, *cur)
 *   NVFP4_OBS_EMA:            *state := (1 - decay) * *state + decay * *cur
 *                             (each product and the sum rounded; 1 - decay in fp32)
 * A negative *state (the -1 initial buffer value) means "no observation yet":
 * the update then stores *cur for either mode.  The updated state is the amax
 * to pass as amax_in when fake-quantizing the same activation.
 *   state, cur  device fp32, 4-byte aligned (cur may equal state)
 *   decay       EMA weight of the new observation, 0 < decay <= 1; ignored for
 *               the static observer
 * Errors: NULL, ALIGN, ARG (mode not 0/1, decay out of range), HIP.
 */
nvfp4_status nvfp4_observer_update(float* state, const float* cur, int mode, float decay,
                                   void* stream);

/*
 * Workspace calls.  nvfp4_fake_quant and nvfp4_quantize_pack without amax_in
 * clear the amax, run the amax pass (one atomic max per workgroup into the
 * amax), then the quantizing pass: three launches.  The calls below take a
 * caller-owned workspace instead: the amax pass leaves one partial maximum per
 * workgroup there, and every workgroup of the quantizing pass reduces them
 * itself (workgroup 0 stores the amax), so there is no clearing launch and no
 * atomic: two launches, 3-6 us less on 32-112 MB tensors.  Same results, bit
 * for bit.  (Rows whose length is not a multiple of 16 take one more launch,
 * which reduces the partials before the quantizing pass.)
 *
 *   workspace  device memory of NVFP4_WORKSPACE_BYTES bytes, 256-byte aligned,
 *              owned by the caller.  Its contents on entry do not matter and are
 *              undefined afterwards; it must not overlap any other argument.  A
 *              call uses it until its last kernel ends: calls that share one
 *              workspace must be ordered (one stream, or events), or they race.
 */
#define NVFP4_WORKSPACE_BYTES 2304

/*
 * nvfp4_fake_quant_ws -- nvfp4_fake_quant(x) with amax_in = NULL: the same y;
 * amax_out (device fp32, or NULL to skip it) receives max|x|.  x and y as for
 * nvfp4_fake_quant (y == x allowed).
 * Errors: SHAPE, NULL, ALIGN, OVERLAP, HIP.
 */
nvfp4_status nvfp4_fake_quant_ws(const void* x, void* y, int64_t rows, int64_t cols,
                                 float* amax_out, void* workspace, void* stream);

/*
 * nvfp4_quantize_pack_ws -- nvfp4_quantize_pack(x) with amax_in = NULL: the same
 * packed, scales and global_scale; amax_out may be NULL.
 * Errors: SHAPE, NULL, ALIGN, OVERLAP, HIP.
 */
nvfp4_status nvfp4_quantize_pack_ws(const void* x, int64_t rows, int64_t cols, float* amax_out,
                                    uint8_t* packed, uint8_t* scales, float* global_scale,
                                    void* workspace, void* stream);

/*
 * nvfp4_fake_quant_group_ws -- nvfp4_fake_quant_group with amax_in = NULL for a
 * group of at most NVFP4_AMAX_GROUP_MAX tensors (fused siblings): the same ys;
 * amax_out (or NULL) receives the shared amax.  Members as for
 * nvfp4_fake_quant_group.
 * Errors: NULL, SHAPE, ARG (n < 1 or n > NVFP4_AMAX_GROUP_MAX), ALIGN, OVERLAP, HIP.
 */
nvfp4_status nvfp4_fake_quant_group_ws(const void* const* xs, void* const* ys, const int64_t* rows,
                                       const int64_t* cols, int n, float* amax_out, void* workspace,
                                       void* stream);

/*
 * nvfp4_observe_fake_quant -- the activation step of a W4A4 layer with one or
 * two observers, as one call (verl QATLinear page, section 5: the step's amax
 * updates the observer, and the activation is fake-quantized with the updated
 * state):
 *   *cur     := max|x|                      (as nvfp4_amax)
 *   *state_i := one nvfp4_observer_update step of *state_i on *cur
 *   y_i      := nvfp4_fake_quant(x) with amax_in = the new *state_i
 * With two observers x is read once for both outputs.  The results are those
 * of the separate calls, bit for bit.
 *
 *   x               device bf16 [rows, cols], 16-byte aligned
 *   cur             device fp32, 4-byte aligned: receives the step amax
 *   state0, y0      first observer state (device fp32, 4-byte aligned) and its
 *                   output (device bf16 [rows, cols], 16-byte aligned; y0 == x
 *                   allowed)
 *   state1, y1      second observer and its output, or both NULL for one
 *                   observer (y1 == x allowed when y0 != x)
 *   mode_i, decay_i as for nvfp4_observer_update
 *   workspace       as for the workspace calls above (NVFP4_WORKSPACE_BYTES,
 *                   256-byte aligned, caller-owned, contents irrelevant)
 * Launches: the amax pass (partial maxima into the workspace, and a copy of
 * the states), then the fake-quant pass, whose every workgroup reduces the
 * partials and steps the observers from the copied states (workgroup 0 stores
 * *cur and the new states).  Rows whose length is not a multiple of 16, and
 * rows == 0, take a one-workgroup launch for the reduction and the steps in
 * between.
 * x, y0 and y1 may be NULL when rows == 0; the states still step on *cur = +0.
 * The amax is the local one: a data-parallel caller that all-reduces the step
 * amax before the observer update uses the separate calls instead.
 * Errors: SHAPE, NULL, ALIGN, OVERLAP, ARG (bad mode or decay, or y1 without
 * state1), HIP.
 */
nvfp4_status nvfp4_observe_fake_quant(const void* x, int64_t rows, int64_t cols, float* cur,
                                      float* state0, int mode0, float decay0, void* y0,
                                      float* state1, int mode1, float decay1, void* y1,
                                      void* workspace, void* stream);

/*
 * MXFP4 variant (VideoX-Fun page, module constants: the block-size comment, which
 * names 32-element blocks with a single-precision scale as the MXFP4 form).
 * Taken literally: blocks of NVFP4_MX_BLOCK = 32 consecutive elements of one row
 * (a row is zero-padded to whole blocks), one binary32 scale per block and no
 * per-tensor factor:
 *   s    = block_amax / 6                      (binary32, stored as is; 0 for a zero block)
 *   q    = x / max(s, 1e-12);  idx = E2M1 round-to-nearest-even of min(|q|, 6)
 *   code = idx | 8 * (q < 0)
 *   fake-quant / unpack output = bf16_RNE(LUT[code] * s)
 * (The OCP MXFP4 format stores a power-of-two E8M0 scale; the page's flavour keeps
 * the scale in fp32, and that is what these calls do.)  No amax pass: one launch
 * per call.  nbr = ceil(cols / 32) blocks per row.
 */
#define NVFP4_MX_BLOCK 32

/*
 * nvfp4_mx_fake_quant -- bf16 [rows, cols] -> bf16 [rows, cols] MXFP4 fake-quant.
 *   x, y  device bf16, 16-byte aligned; y == x (exact in-place) is allowed.
 * Errors: SHAPE, NULL, ALIGN, OVERLAP, HIP.
 */
nvfp4_status nvfp4_mx_fake_quant(const void* x, void* y, int64_t rows, int64_t cols, void* stream);

/*
 * nvfp4_mx_quantize_pack -- bf16 [rows, cols] -> packed MXFP4.
 *   packed  device uint8 [rows, 16 * nbr], 16-byte aligned: byte i of a row holds
 *           the code of (padded) column 2i in its low nibble and of 2i + 1 in its
 *           high nibble; padding columns get code 0
 *   scales  device float [rows, nbr], 4-byte aligned: the binary32 block scales
 * Outputs must not overlap x or each other.
 * Errors: SHAPE, NULL, ALIGN, OVERLAP, HIP.
 */
nvfp4_status nvfp4_mx_quantize_pack(const void* x, int64_t rows, int64_t cols, uint8_t* packed, float* scales,
                                    void* stream);

/*
 * nvfp4_mx_dequant_unpack -- packed MXFP4 -> bf16 [rows, cols] (LUT[code] * s,
 * rounded to bf16).  Layouts as nvfp4_mx_quantize_pack writes them; packed
 * 16-byte aligned, scales 4-byte aligned, y 16-byte aligned and not overlapping
 * the inputs.
 * Errors: SHAPE, NULL, ALIGN, OVERLAP, HIP.
 */
nvfp4_status nvfp4_mx_dequant_unpack(const uint8_t* packed, const float* scales, int64_t rows, int64_t cols,
                                     void* y, void* stream);

/*
 * nvfp4_fake_quant_noalloc -- nvfp4_fake_quant_ws without a workspace argument,
 * for callers that cannot allocate device memory at all (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  Same y and
 * amax_out as nvfp4_fake_quant_ws, bit for bit; x, y and amax_out as there.
 *
 * The workspace is a library-owned device array of NVFP4_WORKSPACE_BYTES bytes:
 * one per GPU, created with the library's code on that GPU and held until the
 * process ends.  Its device address is looked up on the first call on each GPU
 * (the GPU of `stream`); the call itself never allocates or frees memory.  The
 * array's contents carry over from call to call and nothing in it needs to
 * start at zero.  Its size does not grow with the tensor (the amax pass leaves
 * at most 512 partial maxima there), so every shape nvfp4_fake_quant_ws accepts
 * is accepted here; no other size limit applies.
 * Every call on one GPU shares that GPU's array: calls on one GPU whose work
 * overlaps in time (two streams, or host threads with their own streams) race
 * and give undefined results.  Order them on one stream, or use the _ws call
 * with a workspace each.
 * Errors: SHAPE, NULL, ALIGN, OVERLAP, ARG (more than 64 GPUs), HIP (including
 * a failed address lookup).
 */
nvfp4_status nvfp4_fake_quant_noalloc(const void* x, void* y, int64_t rows, int64_t cols, float* amax_out,
                                      void* stream);

/* Human-readable name of a status code (static storage, never NULL). */
const char* nvfp4_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
