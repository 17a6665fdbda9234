// libnvfp4 -- NVFP4 two-level block quantization for AMD Instinct MI355X (gfx950).
//
// What is computed is stated in include/nvfp4.h; it follows the VideoX-Fun page
// "videox_fun/utils/fp4_optimization.py" (quantize_weight_to_float4,
// dequantize_weight_from_float4, _float4_round) and the verl tutorial page
// "linear.py -- QATLinear" (sections 1, 4 and 5).  This file is written for
// CDNA4 from that description; it follows neither page's code.
//
// Design
// ------
// * The quantizing kernels stream HBM (2-6 bytes per element) with a few dozen
//   lane ops per element; the limits are HBM bandwidth and the VALU issue rate.
// * Lanes 2k and 2k+1 hold the two halves of a 16-element block, so every load
//   and store is contiguous across a wave; the block max combines the lane's
//   packed 16-bit max with its partner's through one DPP permute.
// * Element codes: q' = fl(x * r), r = 1 / sq, through the gfx950 FP4
//   converter wherever that is provably the same code as the correctly rounded
//   quotient fl(x / sq) for every bf16 input (a per-scale-byte certificate);
//   otherwise integer compares against exact decision thresholds ("Decision
//   thresholds" below).  Everything that depends only on the E4M3 scale byte S
//   (the multiplier, the decoded scale, the thresholds, the certificate) is
//   tabulated once per workgroup for all 128 bytes in a 4 KB LDS table, so a
//   block costs one scale computation and one LDS lookup.
// * Workgroups walk the tensor with a grid stride, which amortises the table
//   build over many blocks.
// * The per-tensor amax is a separate streaming pass.  The plain calls reduce
//   it with one atomic max per workgroup and the quantizing kernels read the
//   result from device memory; the workspace calls leave one partial maximum
//   per workgroup in the workspace, and every quantizing workgroup reduces them
//   itself.  Either way a fused call never returns to the host.
// * The linear layer over a packed weight is the one dense contraction: there
//   the weight is decoded in registers into bf16 MFMA operands.
//
// Decision thresholds
// -------------------
// For a block divisor sq > 0 the correctly rounded quotient fl(|x| / sq) does
// not decrease as |x| grows, so each of the seven decisions "the quotient
// passes boundary b" holds exactly for |x| from some threshold upward.  Every
// boundary (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5) has a zero last significand
// bit, so under round-to-nearest-even
//     fl(z) >  b   <=>  z >  b + ulp(b)/2        (the tie rounds back to b)
//     fl(z) >= b   <=>  z >= b - ulp_below(b)/2  (the tie rounds up to b)
// and with z = |x| / sq the right-hand sides become |x| > B * sq with B a
// 25-bit constant.  B * sq (25 x 24 bits) is exact in binary64.  Since |x| is a
// bf16 value, "|x| > T" is "bits(|x|) >= bits of the first bf16 above T",
// and "|x| >= T" is "bits(|x|) >= bits of the first bf16 at or above T", both
// compared as 15-bit integers.  The sign of the code is set when x < 0 and
// the quotient does not underflow to zero: |x| / sq > 2^-150.
// The seven sorted thresholds are searched in three packed 16-bit steps.
//
// Files
// -----
// config.hpp   launch shapes, cache hints, constants
// device.hpp   packed 16-bit helpers, memory hints, number formats, the
//              per-scale-byte table, half-block codes and outputs
// kernels.hpp  amax, fake-quant (single, dual, group), quantize-pack,
//              dequant-unpack, the ragged-row kernels, the observer steps
// linear.hpp   the linear layer over a packed weight (MFMA)
// mx.hpp       the MXFP4 variant (32-element blocks, binary32 block scales)
// nvfp4.hip    host helpers (launch shapes, argument checks) and the C ABI

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <atomic>
#include <mutex>

#include "nvfp4.h"
#include "kernels.hpp"
#include "linear.hpp"
#include "mx.hpp"

namespace {

// ---------------------------------------------------------------- host helpers

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool overlap(const void* a, uint64_t na, const void* b, uint64_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return na && nb && x < y + nb && y < x + na;
}

struct Matrix {
    int64_t numel;      // rows * cols
    int64_t nbr;        // blocks per row, ceil(cols / 16)
    int64_t nblocks;    // rows * nbr
    bool ragged;        // cols % 16 != 0
};

nvfp4_status check_matrix(int64_t rows, int64_t cols, Matrix* m)
{
    if (rows < 0 || cols < 1)
        return NVFP4_ERR_SHAPE;
    const int64_t nbr = (cols + 15) / 16;
    if (rows > 0 && nbr > (INT64_MAX / 64) / rows)      // padded bytes stay far from overflow
        return NVFP4_ERR_SHAPE;
    m->numel = rows * cols;
    m->nbr = nbr;
    m->nblocks = rows * nbr;
    m->ragged = cols % 16 != 0;
    return NVFP4_OK;
}

constexpr int kRaggedWgPerCu = 32;

// Devices whose properties (CU count, scratch address) the library caches.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

// Compute units of the current device, queried once per device.
int compute_units()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return 256;
    int cus = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cus == 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        g_cu_count[dev].store(cus, std::memory_order_relaxed);
    }
    return cus;
}

unsigned persistent_grid(int64_t items, int64_t items_per_wg, int wg_per_cu)
{
    const int cus = compute_units();
    const int64_t need = (items + items_per_wg - 1) / items_per_wg;
    const int64_t cap = (int64_t)cus * wg_per_cu;
    return (unsigned)(need < 1 ? 1 : (need < cap ? need : cap));
}

nvfp4_status launched()
{
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

// The amax pass's description of up to NVFP4_AMAX_GROUP_MAX tensors; *chunks
// receives the number of chunks it walks.
AmaxGroup amax_group(const void* const* xs, const int64_t* numels, int n, int64_t* chunks,
                     int64_t alloc_bytes = NVFP4_AMAX_ALLOC_BYTES)
{
    AmaxGroup g{};
    constexpr int64_t kChunk = (int64_t)kThreads * kAmaxUnroll;
    int64_t c = 0;
    g.count = n;
    for (int i = 0; i < n; ++i) {
        g.vec[i] = static_cast<const uint4*>(xs[i]);
        g.nvec[i] = numels[i] / 8;
        g.tail[i] = static_cast<const uint16_t*>(xs[i]) + (numels[i] & ~(int64_t)7);
        g.ntail[i] = (int32_t)(numels[i] & 7);
        c += (g.nvec[i] + kChunk - 1) / kChunk;
        g.chunk_end[i] = c;
    }
    // Only the last alloc_bytes of the group are read with allocating loads: that
    // is what the Infinity Cache still holds when the quantizing pass over the same
    // tensor gets there; the rest streams past the caches.
    const int64_t alloc_chunks = alloc_bytes / (kChunk * 16);
    g.alloc_from = c > alloc_chunks ? c - alloc_chunks : 0;
    *chunks = c;
    return g;
}

// Enqueue max|x| of up to NVFP4_AMAX_GROUP_MAX tensors into *amax (atomic max).
nvfp4_status enqueue_amax(const void* const* xs, const int64_t* numels, int n, float* amax,
                          hipStream_t stream, int64_t alloc_bytes = NVFP4_AMAX_ALLOC_BYTES)
{
    int64_t chunks;
    const AmaxGroup g = amax_group(xs, numels, n, &chunks, alloc_bytes);
    k_amax<false><<<persistent_grid(chunks, 1, NVFP4_AMAX_WG_PER_CU), kThreads, 0, stream>>>(g, amax, nullptr);
    return launched();
}

// Collects non-empty tensors and enqueues one amax launch per
// NVFP4_AMAX_GROUP_MAX of them.
struct AmaxBatch {
    const void* x[NVFP4_AMAX_GROUP_MAX];
    int64_t n[NVFP4_AMAX_GROUP_MAX];
    int k = 0;

    nvfp4_status add(const void* p, int64_t numel, float* amax, hipStream_t s)
    {
        if (numel == 0)
            return NVFP4_OK;
        x[k] = p;
        n[k] = numel;
        return ++k == NVFP4_AMAX_GROUP_MAX ? flush(amax, s) : NVFP4_OK;
    }
    nvfp4_status flush(float* amax, hipStream_t s)
    {
        const int c = k;
        k = 0;
        return c ? enqueue_amax(x, n, c, amax, s) : NVFP4_OK;
    }
};

// *amax := 0, so that the atomic maxima of the launches that follow start clean.
nvfp4_status enqueue_reset(float* amax, hipStream_t s)
{
    k_set_scalar<<<1, 1, 0, s>>>(amax, 0.0f);
    return launched();
}

nvfp4_status enqueue_amax_one(const void* x, int64_t numel, float* amax, hipStream_t stream,
                              int64_t alloc_bytes = NVFP4_AMAX_ALLOC_BYTES)
{
    nvfp4_status st = enqueue_reset(amax, stream);
    if (st != NVFP4_OK || numel == 0)
        return st;
    return enqueue_amax(&x, &numel, 1, amax, stream, alloc_bytes);
}

// Workgroups per CU of a quantizing pass over nhalves half blocks.
int quant_wg_per_cu(int64_t nhalves, int mid, int large)
{
    return nhalves * 16 < NVFP4_MID_BYTES ? mid : large;
}

// Ragged rows take the half-block kernels (32-bit half indices); from
// NVFP4_HALF_ROWS_MAX_BLOCKS blocks on, the one-lane-per-block kernels.
bool half_rows(int64_t cols, const Matrix& m)
{
    (void)cols;
    return m.ragged && m.nblocks < (int64_t)NVFP4_HALF_ROWS_MAX_BLOCKS;
}

HalfRows half_rows_of(const void* x, int64_t cols, const Matrix& m)
{
    return HalfRows{static_cast<const uint16_t*>(x), cols, (uint32_t)(2 * m.nbr), 2 * m.nblocks};
}

// Workgroups per CU of the two-output pass over nhalves half blocks.
int dual_wg_per_cu(int64_t nhalves)
{
    return quant_wg_per_cu(nhalves, NVFP4_DUAL_MID_WG_PER_CU, NVFP4_FQ_WG_PER_CU);
}

// Bytes at the end of the amax pass in front of a quantizing pass that are read
// with allocating loads, for bytes of input (mid: the size below NVFP4_MID_BYTES).
int64_t amax_alloc_bytes(int64_t bytes, int64_t mid)
{
    return bytes < NVFP4_MID_BYTES ? mid : NVFP4_AMAX_ALLOC_BYTES;
}

// One fake-quant launch of a single tensor with its amax from src (partials
// only for rows of whole blocks).
nvfp4_status enqueue_fake_quant(const void* x, void* y, int64_t cols, const Matrix& m, const AmaxIn& src,
                                hipStream_t s)
{
    if (m.numel == 0)
        return NVFP4_OK;
    const float* a = src.amax[0];                  // the one-lane-per-block kernels take a direct amax
    if (half_rows(cols, m)) {
        const HalfRows g = half_rows_of(x, cols, m);
        const dim3 grid(persistent_grid(g.nhalves, (int64_t)kThreads * kUnroll,
                                        quant_wg_per_cu(g.nhalves, NVFP4_FQ_MID_WG_PER_CU, NVFP4_FQ_WG_PER_CU)));
        uint16_t* yh = static_cast<uint16_t*>(y);
        if (cols % 2 == 0 && src.partials)
            k_fake_quant_rows<true, false><<<grid, kThreads, 0, s>>>(g, yh, src);
        else if (cols % 2 == 0)
            k_fake_quant_rows<false, false><<<grid, kThreads, 0, s>>>(g, yh, src);
        else if (src.partials)
            k_fake_quant_rows<true, true><<<grid, kThreads, 0, s>>>(g, yh, src);
        else
            k_fake_quant_rows<false, true><<<grid, kThreads, 0, s>>>(g, yh, src);
        return launched();
    }
    if (m.ragged) {
        const RaggedShape g{cols, m.nbr, m.nblocks};
        k_fake_quant_ragged<<<persistent_grid(m.nblocks, kThreads, kRaggedWgPerCu), kThreads, 0, s>>>(
            static_cast<const uint16_t*>(x), static_cast<uint16_t*>(y), g, a);
        return launched();
    }
    const int64_t nh = 2 * m.nblocks;
    const dim3 grid(persistent_grid(nh, (int64_t)kThreads * kUnroll,
                                    quant_wg_per_cu(nh, NVFP4_FQ_MID_WG_PER_CU, NVFP4_FQ_WG_PER_CU)));
    if (src.partials)
        k_fake_quant<true><<<grid, kThreads, 0, s>>>(static_cast<const uint4*>(x), static_cast<uint4*>(y), nh, src);
    else
        k_fake_quant<false><<<grid, kThreads, 0, s>>>(static_cast<const uint4*>(x), static_cast<uint4*>(y), nh, src);
    return launched();
}

// The same with a device amax.
nvfp4_status enqueue_fake_quant(const void* x, void* y, int64_t cols, const Matrix& m, const float* a,
                                hipStream_t s)
{
    return enqueue_fake_quant(x, y, cols, m, AmaxIn{{a, nullptr}}, s);
}

// One quantize-pack launch of a single tensor (also for an empty one: it still
// writes the global scale).
nvfp4_status enqueue_quantize_pack(const void* x, int64_t cols, const Matrix& m, uint8_t* packed, uint8_t* scales,
                                   float* global_scale, const AmaxIn& src, hipStream_t s)
{
    const float* a = src.amax[0];                  // the one-lane-per-block kernel takes a direct amax
    if (half_rows(cols, m)) {
        const HalfRows g = half_rows_of(x, cols, m);
        const dim3 grid(persistent_grid(g.nhalves, (int64_t)kThreads * kUnroll,
                                        quant_wg_per_cu(g.nhalves, NVFP4_QP_MID_WG_PER_CU, NVFP4_QP_WG_PER_CU)));
        uint32_t* pv = reinterpret_cast<uint32_t*>(packed);
        if (cols % 2 == 0 && src.partials)
            k_quantize_pack_rows<true, false><<<grid, kThreads, 0, s>>>(g, pv, scales, global_scale, src);
        else if (cols % 2 == 0)
            k_quantize_pack_rows<false, false><<<grid, kThreads, 0, s>>>(g, pv, scales, global_scale, src);
        else if (src.partials)
            k_quantize_pack_rows<true, true><<<grid, kThreads, 0, s>>>(g, pv, scales, global_scale, src);
        else
            k_quantize_pack_rows<false, true><<<grid, kThreads, 0, s>>>(g, pv, scales, global_scale, src);
        return launched();
    }
    if (m.ragged) {
        const RaggedShape g{cols, m.nbr, m.nblocks};
        k_quantize_pack_ragged<<<persistent_grid(m.nblocks, kThreads, kRaggedWgPerCu), kThreads, 0, s>>>(
            static_cast<const uint16_t*>(x), reinterpret_cast<uint2*>(packed), scales, global_scale, g, a);
        return launched();
    }
    const int64_t nh = 2 * m.nblocks;
    const dim3 grid(persistent_grid(nh, (int64_t)kThreads * kUnroll,
                                    quant_wg_per_cu(nh, NVFP4_QP_MID_WG_PER_CU, NVFP4_QP_WG_PER_CU)));
    const uint4* xv = static_cast<const uint4*>(x);
    uint32_t* pv = reinterpret_cast<uint32_t*>(packed);
    if (src.partials)
        k_quantize_pack<true><<<grid, kThreads, 0, s>>>(xv, pv, scales, global_scale, nh, src);
    else
        k_quantize_pack<false><<<grid, kThreads, 0, s>>>(xv, pv, scales, global_scale, nh, src);
    return launched();
}

nvfp4_status enqueue_quantize_pack(const void* x, int64_t cols, const Matrix& m, uint8_t* packed, uint8_t* scales,
                                   float* global_scale, const float* a, hipStream_t s)
{
    return enqueue_quantize_pack(x, cols, m, packed, scales, global_scale, AmaxIn{{a, nullptr}}, s);
}

// The workspace of the calls that take one: the amax (when the caller asks
// for none) at byte 0, the amax pass's partial maxima from byte kPartialsOffset.
constexpr int64_t kPartialsOffset = 256;
constexpr int kMaxPartials = NVFP4_MAX_PARTIALS;
static_assert(kPartialsOffset + 4 * kMaxPartials <= NVFP4_WORKSPACE_BYTES, "partials fit the workspace");
static_assert(kMaxPartials >= NVFP4_AMAX_WG_PER_CU * 256, "the workspace holds a partial per amax workgroup");

// Enqueue the amax of up to NVFP4_AMAX_GROUP_MAX tensors through the workspace:
// the amax pass in partials mode, then their reduction into *amax, followed by
// nobs observer steps on it.  An all-empty group gets one workgroup, which stores
// a zero partial.
// The amax pass alone, in partials mode: *src gets the partials and their count,
// and, with nobs observers, their arguments and the states as the pass copies
// them into the workspace (at byte kPriorOffset).
constexpr int64_t kPriorOffset = 16;
static_assert(kPriorOffset >= 4 && kPriorOffset + 8 <= kPartialsOffset, "workspace layout");

nvfp4_status enqueue_amax_partials(const void* const* xs, const int64_t* numels, int n, void* ws,
                                   hipStream_t stream, AmaxIn* src, const ObserverArgs& obs = ObserverArgs{},
                                   int nobs = 0, int64_t alloc_bytes = NVFP4_AMAX_ALLOC_BYTES)
{
    int64_t chunks;
    AmaxGroup g = amax_group(xs, numels, n, &chunks, alloc_bytes);
    unsigned grid = persistent_grid(chunks, 1, NVFP4_AMAX_WG_PER_CU);
    if (grid > (unsigned)kMaxPartials)
        grid = (unsigned)kMaxPartials;
    uint32_t* partials = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + kPartialsOffset);
    float* prior = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + kPriorOffset);
    for (int i = 0; i < nobs; ++i)
        g.snap_from[i] = obs.state[i];
    g.snap_to = prior;
    g.nsnap = nobs;
    k_amax<true><<<grid, kThreads, 0, stream>>>(g, nullptr, partials);
    *src = AmaxIn{};
    src->partials = partials;
    src->count = (int)grid;
    src->obs = obs;
    src->nobs = nobs;
    src->prior = prior;
    return launched();
}

nvfp4_status enqueue_amax_ws(const void* const* xs, const int64_t* numels, int n, void* ws, float* amax,
                             hipStream_t stream, const ObserverArgs& obs = ObserverArgs{}, int nobs = 0)
{
    AmaxIn src{};
    if (enqueue_amax_partials(xs, numels, n, ws, stream, &src) != NVFP4_OK)
        return NVFP4_ERR_HIP;
    k_amax_finish<<<1, kThreads, 0, stream>>>(src.partials, src.count, amax, obs, nobs);
    return launched();
}

// Where a workspace call keeps the amax: the caller's amax_out, else the workspace.
float* ws_amax(void* ws, float* amax_out) { return amax_out ? amax_out : static_cast<float*>(ws); }

// Collects tensors whose rows are whole blocks and enqueues one group launch
// per NVFP4_AMAX_GROUP_MAX of them.
struct FakeQuantBatch {
    FqGroup g{};
    int64_t chunks = 0;

    nvfp4_status add(const void* x, void* y, int64_t nblocks, const AmaxIn& src, hipStream_t s)
    {
        constexpr int64_t kChunk = (int64_t)kThreads * kUnroll;
        const int k = g.count;
        g.x[k] = static_cast<const uint4*>(x);
        g.y[k] = static_cast<uint4*>(y);
        g.nhalves[k] = 2 * nblocks;
        chunks += (2 * nblocks + kChunk - 1) / kChunk;
        g.chunk_end[k] = chunks;
        return ++g.count == NVFP4_AMAX_GROUP_MAX ? flush(src, s) : NVFP4_OK;
    }
    nvfp4_status flush(const AmaxIn& src, hipStream_t s)
    {
        if (g.count == 0)
            return NVFP4_OK;
        constexpr int64_t kChunk = (int64_t)kThreads * kUnroll;
        const dim3 grid(persistent_grid(chunks, 1, quant_wg_per_cu(chunks * kChunk, NVFP4_FQ_MID_WG_PER_CU,
                                                                   NVFP4_FQ_WG_PER_CU)));
        if (src.partials)
            k_fake_quant_group<true><<<grid, kThreads, 0, s>>>(g, src);
        else
            k_fake_quant_group<false><<<grid, kThreads, 0, s>>>(g, src);
        g = FqGroup{};
        chunks = 0;
        return launched();
    }
};

// One launch of the linear kernel with MT x NT MFMA tiles per workgroup, W
// waves, KS-wide K steps.
template <int MT, int NT, int W, int KS>
nvfp4_status enqueue_linear(const void* x, int64_t m, int64_t k, const uint8_t* packed,
                            const uint8_t* scales, const float* gs, int64_t n, const void* bias, void* y,
                            hipStream_t s)
{
    const dim3 grid((unsigned)((n + 16 * NT - 1) / (16 * NT)), (unsigned)((m + 16 * MT - 1) / (16 * MT)));
    const size_t partial_bytes = (size_t)(W - 1) * lin_partial_tiles<MT, NT, W>() * NT * 64 * sizeof(f32x4);
    const size_t scale_bytes = (size_t)16 * NT * (k / 16);
    // the scale rows go to LDS when they fit in the 64 KB a workgroup may always use
    if (NVFP4_LIN_SCALES_LDS && scale_bytes <= kLinLdsBudget) {
        const size_t lds = scale_bytes > partial_bytes ? scale_bytes : partial_bytes;
        k_linear<MT, NT, W, KS, true><<<grid, 64 * W, lds, s>>>(
            static_cast<const uint16_t*>(x), m, k, reinterpret_cast<const uint32_t*>(packed), scales, gs, n,
            static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(y));
    } else {
        k_linear<MT, NT, W, KS, false><<<grid, 64 * W, partial_bytes, s>>>(
            static_cast<const uint16_t*>(x), m, k, reinterpret_cast<const uint32_t*>(packed), scales, gs, n,
            static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(y));
    }
    return launched();
}

// K step: 256 wide (fewer, wider loads) for one 16-row tile of x and at most
// four weight tiles, else 128 wide (fewer registers).  The waves split K: 8 for
// one 16-row tile of x (more loads in flight per CU; 33 vs 38 us for one row of
// x on the c5 weight), else 4 (8 waves of 2-4 x tiles spill registers, the
// double-buffered x operands: 64 rows of x on the c5 weight took 211 us against
// 59; 16 waves spill for one tile too).
template <int MT, int NT>
nvfp4_status enqueue_linear_w(const void* x, int64_t m, int64_t k, const uint8_t* packed,
                              const uint8_t* scales, const float* gs, int64_t n, const void* bias, void* y,
                              hipStream_t s)
{
    constexpr int kKS = NVFP4_LIN_KS ? NVFP4_LIN_KS : (MT == 1 && NT <= 4 ? 256 : 128);
    constexpr int kW = NVFP4_LIN_W ? NVFP4_LIN_W : (MT == 1 ? 8 : 4);
    return enqueue_linear<MT, NT, kW, kKS>(x, m, k, packed, scales, gs, n, bias, y, s);
}

// Weight tiles per workgroup.  A weight of N rows is N / 16 tiles; when that is
// 256 c for c <= 8 (N a multiple of 4096, as the widths of transformer layers
// usually are), c tiles per workgroup give every CU of the 256 exactly one
// workgroup, which measured best for 16 to 64 rows of x (and within 3% for one
// row).  Otherwise: 4, 2 or 1 tiles, the largest that still makes 256
// workgroups.
template <int MT>
nvfp4_status enqueue_linear_mt(const void* x, int64_t m, int64_t k, const uint8_t* packed,
                               const uint8_t* scales, const float* gs, int64_t n, const void* bias, void* y,
                               hipStream_t s)
{
#define NVFP4_LIN_ARGS x, m, k, packed, scales, gs, n, bias, y, s
    if (NVFP4_LIN_NT > 0)
        return enqueue_linear_w<MT, NVFP4_LIN_NT == 0 ? 1 : NVFP4_LIN_NT>(NVFP4_LIN_ARGS);
    const int64_t gy = (m + 16 * MT - 1) / (16 * MT);
    if (gy == 1 && n % 4096 == 0) {
        switch (n / 4096) {
        case 1: return enqueue_linear_w<MT, 1>(NVFP4_LIN_ARGS);
        case 2: return enqueue_linear_w<MT, 2>(NVFP4_LIN_ARGS);
        case 3: return enqueue_linear_w<MT, 3>(NVFP4_LIN_ARGS);
        case 4: return enqueue_linear_w<MT, 4>(NVFP4_LIN_ARGS);
        case 5: return enqueue_linear_w<MT, 5>(NVFP4_LIN_ARGS);
        case 6: return enqueue_linear_w<MT, 6>(NVFP4_LIN_ARGS);
        case 7: return enqueue_linear_w<MT, 7>(NVFP4_LIN_ARGS);
        case 8: return enqueue_linear_w<MT, 8>(NVFP4_LIN_ARGS);
        default: break;
        }
    }
    if (((n + 63) / 64) * gy >= 256)
        return enqueue_linear_w<MT, 4>(NVFP4_LIN_ARGS);
    if (((n + 31) / 32) * gy >= 256)
        return enqueue_linear_w<MT, 2>(NVFP4_LIN_ARGS);
    return enqueue_linear_w<MT, 1>(NVFP4_LIN_ARGS);
#undef NVFP4_LIN_ARGS
}

// One launch of the tiled linear kernel (many rows of x).
template <int MW, int NW>
nvfp4_status enqueue_linear_tiled(const void* x, int64_t m, int64_t k, const uint8_t* packed,
                                    const uint8_t* scales, const float* gs, int64_t n, const void* bias, void* y,
                                    hipStream_t s)
{
    const dim3 grid((unsigned)((m + 32 * MW - 1) / (32 * MW)),
                    (unsigned)((n + 32 * NW * kTileWaves - 1) / (32 * NW * kTileWaves)));
    if (k % 64 == 0) {
        constexpr size_t lds = (size_t)2 * 32 * MW * (64 + 8) * 2;
        k_linear_tiled<MW, NW, 64><<<grid, 64 * kTileWaves, lds, s>>>(
            static_cast<const uint16_t*>(x), m, k, packed, scales, gs, n, static_cast<const uint16_t*>(bias),
            static_cast<uint16_t*>(y));
    } else {
        constexpr size_t lds = (size_t)2 * 32 * MW * (32 + 8) * 2;
        k_linear_tiled<MW, NW, 32><<<grid, 64 * kTileWaves, lds, s>>>(
            static_cast<const uint16_t*>(x), m, k, packed, scales, gs, n, static_cast<const uint16_t*>(bias),
            static_cast<uint16_t*>(y));
    }
    return launched();
}

// One launch of the LDS-staged linear kernel (K a multiple of 64) with a tile of
// LdsTile<W, WM, TM, TN>.  Its LDS can exceed the 64 KB a kernel gets by default,
// so the limit is raised once per device and shape.
template <int W, int WM, int TM, int TN, int KG = 1>
nvfp4_status enqueue_linear_lds(const void* x, int64_t m, int64_t k, const uint8_t* packed, const uint8_t* scales,
                                const float* gs, int64_t nb, int64_t ne, int64_t n, const void* bias, void* y,
                                hipStream_t s)
{
    // weight rows [nb, ne) of the n: their codes, scales, bias and columns of y
    using Tile = LdsTile<W, WM, TM, TN>;
    constexpr int WD = 4;
    if ((k / kLdsK) % KG != 0)
        return NVFP4_ERR_SHAPE;
    static std::atomic<int> ready[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return NVFP4_ERR_HIP;
    if (!ready[dev].load(std::memory_order_acquire)) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(&k_linear_lds<W, WM, TM, TN, WD, KG>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)(KG * Tile::kBytes)) != hipSuccess)
            return NVFP4_ERR_HIP;
        ready[dev].store(1, std::memory_order_release);
    }
    const int64_t rows = ne - nb;
    const dim3 grid((unsigned)((m + Tile::kM - 1) / Tile::kM), (unsigned)((rows + Tile::kN - 1) / Tile::kN));
    if (grid.y > 65535)
        return NVFP4_ERR_SHAPE;
    k_linear_lds<W, WM, TM, TN, WD, KG><<<grid, 64 * W * KG, KG * Tile::kBytes, s>>>(
        static_cast<const uint16_t*>(x), m, k, packed + nb * (k / 2), scales + nb * (k / 16), gs, rows,
        bias ? static_cast<const uint16_t*>(bias) + nb : nullptr, static_cast<uint16_t*>(y) + nb, n);
    return launched();
}

// CUs the linear layer plans its tile rounds for.
int64_t linear_cus()
{
    return NVFP4_LIN_RETILE_CUS > 0 ? NVFP4_LIN_RETILE_CUS : compute_units();
}

// The 256 x 256 tiles run one workgroup per CU (their LDS fills it), so they run in
// rounds of one tile per CU.  A partial last round leaves CUs idle; instead, the
// weight rows of that round are re-tiled into the narrowest tiles (64 TN rows,
// TN < 4) of which one round covers them, and run as a second launch that takes
// about TN / 4 of a round.  Each output element's sum is the same in either tile.
nvfp4_status enqueue_linear_lds_large(const void* x, int64_t m, int64_t k, const uint8_t* packed,
                                      const uint8_t* scales, const float* gs, int64_t n, const void* bias,
                                      void* y, hipStream_t s)
{
    const int64_t cus = linear_cus();
    const int64_t mt = (m + 255) / 256, tiles = mt * ((n + 255) / 256), whole = tiles / cus * cus;
    if (NVFP4_LIN_RETILE && tiles > cus && whole < tiles && whole % mt == 0) {
        const int64_t split = whole / mt * 256, rest = n - split;
        const int tn = mt * ((rest + 63) / 64) <= cus ? 1 : mt * ((rest + 127) / 128) <= cus ? 2
                     : mt * ((rest + 191) / 192) <= cus ? 3 : 4;
        if (tn < 4) {
            const nvfp4_status st = enqueue_linear_lds<8, 4, 2, 4>(x, m, k, packed, scales, gs, 0, split, n, bias, y, s);
            if (st != NVFP4_OK)
                return st;
            if (tn == 1)
                return enqueue_linear_lds<8, 4, 2, 1>(x, m, k, packed, scales, gs, split, n, n, bias, y, s);
            if (tn == 2)
                return enqueue_linear_lds<8, 4, 2, 2>(x, m, k, packed, scales, gs, split, n, n, bias, y, s);
            return enqueue_linear_lds<8, 4, 2, 3>(x, m, k, packed, scales, gs, split, n, n, bias, y, s);
        }
    }
    return enqueue_linear_lds<8, 4, 2, 4>(x, m, k, packed, scales, gs, 0, n, n, bias, y, s);
}

// A device region an entry point reads or writes.
struct Region {
    const void* p;
    uint64_t bytes;
};

// Outputs must be disjoint from each other and from the inputs, except that an
// output with the start and size of in[0] may be in[0] itself (exact in-place)
// when inplace_ok.  Empty regions overlap nothing.
nvfp4_status check_regions(const Region* in, int nin, const Region* out, int nout, bool inplace_ok)
{
    for (int i = 0; i < nout; ++i) {
        for (int j = 0; j < nin; ++j) {
            const bool same = inplace_ok && j == 0 && out[i].p == in[0].p && out[i].bytes == in[0].bytes;
            if (!same && overlap(out[i].p, out[i].bytes, in[j].p, in[j].bytes))
                return NVFP4_ERR_OVERLAP;
        }
        for (int j = i + 1; j < nout; ++j)
            if (overlap(out[i].p, out[i].bytes, out[j].p, out[j].bytes))
                return NVFP4_ERR_OVERLAP;
    }
    return NVFP4_OK;
}

// Shapes, pointers, alignment and overlaps of the members of a group call:
// every y_i may be x_i itself (exact in-place) and must not touch anything else.
nvfp4_status check_group_members(const void* const* xs, void* const* ys, const int64_t* rows,
                                 const int64_t* cols, int n)
{
    for (int i = 0; i < n; ++i) {
        Matrix m;
        const nvfp4_status st = check_matrix(rows[i], cols[i], &m);
        if (st != NVFP4_OK)
            return st;
        if (m.numel > 0 && (!xs[i] || !ys[i]))
            return NVFP4_ERR_NULL;
    }
    for (int i = 0; i < n; ++i)
        if (!aligned(xs[i], 16) || !aligned(ys[i], 16))
            return NVFP4_ERR_ALIGN;
    for (int i = 0; i < n; ++i) {
        const uint64_t bi = 2 * (uint64_t)(rows[i] * cols[i]);
        for (int j = 0; j < n; ++j) {
            const uint64_t bj = 2 * (uint64_t)(rows[j] * cols[j]);
            if (!(i == j && xs[i] == ys[i]) && overlap(ys[i], bi, xs[j], bj))
                return NVFP4_ERR_OVERLAP;
            if (j > i && overlap(ys[i], bi, ys[j], bj))
                return NVFP4_ERR_OVERLAP;
        }
    }
    return NVFP4_OK;
}

// The fake-quant of every member with the amax from src: members whose rows are
// whole blocks share group launches, ragged ones get a launch each (which needs
// a direct amax, src.amax[0]).
nvfp4_status enqueue_group_fake_quant(const void* const* xs, void* const* ys, const int64_t* rows,
                                      const int64_t* cols, int n, const AmaxIn& src, hipStream_t s)
{
    FakeQuantBatch batch;
    for (int i = 0; i < n; ++i) {
        Matrix m;
        check_matrix(rows[i], cols[i], &m);
        if (m.numel == 0)
            continue;
        const nvfp4_status st = m.ragged ? enqueue_fake_quant(xs[i], ys[i], cols[i], m, src.amax[0], s)
                                         : batch.add(xs[i], ys[i], m.nblocks, src, s);
        if (st != NVFP4_OK)
            return st;
    }
    return batch.flush(src, s);
}

nvfp4_status enqueue_group_fake_quant(const void* const* xs, void* const* ys, const int64_t* rows,
                                      const int64_t* cols, int n, const float* a, hipStream_t s)
{
    return enqueue_group_fake_quant(xs, ys, rows, cols, n, AmaxIn{{a, nullptr}}, s);
}

bool observer_args_ok(int mode, float decay)
{
    if (mode != NVFP4_OBS_STATIC_MINMAX && mode != NVFP4_OBS_EMA)
        return false;
    return mode != NVFP4_OBS_EMA || (decay > 0.0f && decay <= 1.0f);
}


// Shapes, pointers and alignment of the fused fake-quant through a workspace
// (the workspace itself is checked by the caller).
nvfp4_status check_fake_quant_ws(const void* x, const void* y, int64_t rows, int64_t cols, const float* amax_out,
                                 Matrix* m)
{
    const nvfp4_status st = check_matrix(rows, cols, m);
    if (st != NVFP4_OK)
        return st;
    if (m->numel > 0 && (!x || !y))
        return NVFP4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(y, 16) || (amax_out && !aligned(amax_out, 4)))
        return NVFP4_ERR_ALIGN;
    return NVFP4_OK;
}

// The fused fake-quant through the workspace ws: the amax pass into partial
// maxima, then the fake-quant pass, which reduces them itself (rows of whole
// blocks), or the partials reduced by one workgroup first (ragged rows).  The
// partials are written by the amax pass before anything reads them, and the
// pass reads exactly as many as it wrote, so nothing in ws needs clearing.
nvfp4_status enqueue_fake_quant_ws(const void* x, void* y, int64_t cols, const Matrix& m, float* amax_out,
                                   void* ws, hipStream_t s)
{
    if (m.numel == 0)
        return amax_out ? enqueue_reset(amax_out, s) : NVFP4_OK;
    if (!m.ragged || half_rows(cols, m)) {
        AmaxIn src;
        if (enqueue_amax_partials(&x, &m.numel, 1, ws, s, &src, ObserverArgs{}, 0,
                                  amax_alloc_bytes(2 * m.numel, NVFP4_FQ_AMAX_ALLOC_MID)) != NVFP4_OK)
            return NVFP4_ERR_HIP;
        src.store = amax_out;
        return enqueue_fake_quant(x, y, cols, m, src, s);
    }
    float* a = ws_amax(ws, amax_out);
    if (enqueue_amax_ws(&x, &m.numel, 1, ws, a, s) != NVFP4_OK)
        return NVFP4_ERR_HIP;
    return enqueue_fake_quant(x, y, cols, m, a, s);
}

// Shape of an MXFP4 call: blocks of 32 per row, whole-block rows or not.
nvfp4_status check_mx_matrix(int64_t rows, int64_t cols, Matrix* m)
{
    if (rows < 0 || cols < 1)
        return NVFP4_ERR_SHAPE;
    const int64_t nbr = (cols + kMxBlock - 1) / kMxBlock;
    if (rows > 0 && nbr > (INT64_MAX / 128) / rows)
        return NVFP4_ERR_SHAPE;
    m->numel = rows * cols;
    m->nbr = nbr;
    m->nblocks = rows * nbr;
    m->ragged = cols % kMxBlock != 0;
    return NVFP4_OK;
}

}  // namespace

// ---------------------------------------------------------------- library-owned scratch
//
// nvfp4_fake_quant_noalloc runs the workspace form of the fused fake-quant on
// the `scratch` array below instead of a caller's workspace, so it needs no
// memory from its caller or from an allocator.  Each GPU the library runs on
// holds its own copy of the array, at its own address, until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per GPU (with that GPU current) and only
// that address is ever passed to a kernel.  Every call on one GPU shares the
// array, so calls that overlap in time on one GPU race.
static __device__ __align__(256) uint8_t scratch[NVFP4_WORKSPACE_BYTES];

namespace {

static_assert(kPartialsOffset + 4 * (int64_t)kMaxPartials <= (int64_t)sizeof(scratch),
              "the scratch holds the amax pass's partial maxima for any tensor size");

std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_lock;

// The device address of `scratch` on the GPU of `stream`, looked up on the
// first call there.
nvfp4_status scratch_address(hipStream_t stream, void** out)
{
    int dev = -1;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess)
        return NVFP4_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices)
        return NVFP4_ERR_ARG;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_lock);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            int cur = -1;
            if (hipGetDevice(&cur) != hipSuccess)
                return NVFP4_ERR_HIP;
            if (cur != dev && hipSetDevice(dev) != hipSuccess)
                return NVFP4_ERR_HIP;
            const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (cur != dev)
                (void)hipSetDevice(cur);
            if (e != hipSuccess || !p)
                return NVFP4_ERR_HIP;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return NVFP4_OK;
}

}  // namespace

// ---------------------------------------------------------------- C ABI

extern "C" {

const char* nvfp4_strerror(int status)
{
    switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "a required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "bad shape (need rows >= 0 and cols >= 1)";
    case NVFP4_ERR_ALIGN: return "misaligned pointer";
    case NVFP4_ERR_OVERLAP: return "an output overlaps an input or another output";
    case NVFP4_ERR_ARG: return "bad argument (mode, decay or group count)";
    case NVFP4_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
    }
}

nvfp4_status nvfp4_amax(const void* const* xs, const int64_t* numels, int n, float* amax,
                        int accumulate, void* stream)
{
    if (!xs || !numels || !amax)
        return NVFP4_ERR_NULL;
    if (n < 1)
        return NVFP4_ERR_ARG;
    if (!aligned(amax, 4))
        return NVFP4_ERR_ALIGN;
    for (int i = 0; i < n; ++i) {
        if (numels[i] < 0)
            return NVFP4_ERR_SHAPE;
        if (numels[i] > 0 && !xs[i])
            return NVFP4_ERR_NULL;
        if (numels[i] > 0 && !aligned(xs[i], 16))
            return NVFP4_ERR_ALIGN;
        if (overlap(xs[i], 2 * (uint64_t)numels[i], amax, 4))
            return NVFP4_ERR_OVERLAP;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (!accumulate && enqueue_reset(amax, s) != NVFP4_OK)
        return NVFP4_ERR_HIP;
    AmaxBatch batch;
    for (int i = 0; i < n; ++i) {
        const nvfp4_status st = batch.add(xs[i], numels[i], amax, s);
        if (st != NVFP4_OK)
            return st;
    }
    return batch.flush(amax, s);
}

nvfp4_status nvfp4_fake_quant(const void* x, void* y, int64_t rows, int64_t cols,
                              const float* amax_in, float* amax_out, void* stream)
{
    Matrix m;
    nvfp4_status st = check_matrix(rows, cols, &m);
    if (st != NVFP4_OK)
        return st;
    const int64_t n = m.numel;
    if ((n > 0 && (!x || !y)) || (!amax_in && !amax_out))
        return NVFP4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(y, 16) || (amax_in && !aligned(amax_in, 4)) ||
        (!amax_in && !aligned(amax_out, 4)))
        return NVFP4_ERR_ALIGN;
    const uint64_t bytes = 2 * (uint64_t)n;
    if (x != y && overlap(x, bytes, y, bytes))
        return NVFP4_ERR_OVERLAP;
    if (!amax_in && (overlap(amax_out, 4, x, bytes) || overlap(amax_out, 4, y, bytes)))
        return NVFP4_ERR_OVERLAP;
    if (amax_in && overlap(amax_in, 4, y, bytes))
        return NVFP4_ERR_OVERLAP;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    const float* a = amax_in;
    if (!a) {
        st = enqueue_amax_one(x, n, amax_out, s, amax_alloc_bytes(2 * n, NVFP4_FQ_AMAX_ALLOC_MID));
        if (st != NVFP4_OK)
            return st;
        a = amax_out;
    }
    return enqueue_fake_quant(x, y, cols, m, a, s);
}

nvfp4_status nvfp4_fake_quant_group(const void* const* xs, void* const* ys, const int64_t* rows,
                                    const int64_t* cols, int n, const float* amax_in,
                                    float* amax_out, void* stream)
{
    if (!xs || !ys || !rows || !cols)
        return NVFP4_ERR_NULL;
    if (n < 1)
        return NVFP4_ERR_ARG;
    nvfp4_status st = check_group_members(xs, ys, rows, cols, n);
    if (st != NVFP4_OK)
        return st;
    if (!amax_in && !amax_out)
        return NVFP4_ERR_NULL;
    if ((amax_in && !aligned(amax_in, 4)) || (!amax_in && !aligned(amax_out, 4)))
        return NVFP4_ERR_ALIGN;
    for (int i = 0; i < n; ++i) {
        const uint64_t bi = 2 * (uint64_t)(rows[i] * cols[i]);
        if (!amax_in && (overlap(amax_out, 4, xs[i], bi) || overlap(amax_out, 4, ys[i], bi)))
            return NVFP4_ERR_OVERLAP;
        if (amax_in && overlap(amax_in, 4, ys[i], bi))
            return NVFP4_ERR_OVERLAP;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    const float* a = amax_in;
    if (!a) {
        if (enqueue_reset(amax_out, s) != NVFP4_OK)
            return NVFP4_ERR_HIP;
        AmaxBatch amax;
        for (int i = 0; i < n; ++i)
            if ((st = amax.add(xs[i], rows[i] * cols[i], amax_out, s)) != NVFP4_OK)
                return st;
        if ((st = amax.flush(amax_out, s)) != NVFP4_OK)
            return st;
        a = amax_out;
    }
    return enqueue_group_fake_quant(xs, ys, rows, cols, n, a, s);
}

nvfp4_status nvfp4_fake_quant_group_ws(const void* const* xs, void* const* ys, const int64_t* rows,
                                       const int64_t* cols, int n, float* amax_out, void* workspace,
                                       void* stream)
{
    if (!xs || !ys || !rows || !cols || !workspace)
        return NVFP4_ERR_NULL;
    if (n < 1 || n > NVFP4_AMAX_GROUP_MAX)
        return NVFP4_ERR_ARG;
    nvfp4_status st = check_group_members(xs, ys, rows, cols, n);
    if (st != NVFP4_OK)
        return st;
    if (!aligned(workspace, 256) || (amax_out && !aligned(amax_out, 4)))
        return NVFP4_ERR_ALIGN;
    const Region extra[2] = {{workspace, NVFP4_WORKSPACE_BYTES}, {amax_out, amax_out ? 4u : 0u}};
    if (overlap(extra[0].p, extra[0].bytes, extra[1].p, extra[1].bytes))
        return NVFP4_ERR_OVERLAP;
    for (int i = 0; i < n; ++i) {
        const uint64_t bi = 2 * (uint64_t)(rows[i] * cols[i]);
        for (const Region& e : extra)
            if (overlap(e.p, e.bytes, xs[i], bi) || overlap(e.p, e.bytes, ys[i], bi))
                return NVFP4_ERR_OVERLAP;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    int64_t numels[NVFP4_AMAX_GROUP_MAX];
    bool whole_blocks = true, any = false;
    for (int i = 0; i < n; ++i) {
        numels[i] = rows[i] * cols[i];
        any = any || numels[i] > 0;
        whole_blocks = whole_blocks && (numels[i] == 0 || cols[i] % 16 == 0);
    }
    if (any && whole_blocks) {
        // one group launch, which reduces the partials itself and stores the amax
        int64_t total = 0;
        for (int i = 0; i < n; ++i)
            total += 2 * numels[i];
        AmaxIn src;
        if (enqueue_amax_partials(xs, numels, n, workspace, s, &src, ObserverArgs{}, 0,
                                  amax_alloc_bytes(total, NVFP4_FQ_AMAX_ALLOC_MID)) != NVFP4_OK)
            return NVFP4_ERR_HIP;
        src.store = amax_out;
        return enqueue_group_fake_quant(xs, ys, rows, cols, n, src, s);
    }
    float* a = ws_amax(workspace, amax_out);
    if (enqueue_amax_ws(xs, numels, n, workspace, a, s) != NVFP4_OK)
        return NVFP4_ERR_HIP;
    return enqueue_group_fake_quant(xs, ys, rows, cols, n, a, s);
}


nvfp4_status nvfp4_fake_quant_dual(const void* x, int64_t rows, int64_t cols, const float* amax0,
                                   void* y0, const float* amax1, void* y1, void* stream)
{
    Matrix m;
    nvfp4_status st = check_matrix(rows, cols, &m);
    if (st != NVFP4_OK)
        return st;
    if ((m.numel > 0 && (!x || !y0 || !y1)) || !amax0 || !amax1)
        return NVFP4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(y0, 16) || !aligned(y1, 16) || !aligned(amax0, 4) ||
        !aligned(amax1, 4))
        return NVFP4_ERR_ALIGN;
    const uint64_t bytes = 2 * (uint64_t)m.numel;
    if (overlap(y0, bytes, y1, bytes) || (y0 != x && overlap(y0, bytes, x, bytes)) ||
        (y1 != x && overlap(y1, bytes, x, bytes)))
        return NVFP4_ERR_OVERLAP;
    for (const float* a : {amax0, amax1})
        if (overlap(a, 4, y0, bytes) || overlap(a, 4, y1, bytes))
            return NVFP4_ERR_OVERLAP;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (m.numel == 0)
        return NVFP4_OK;
    if (m.ragged) {
        // two passes; an output written in place goes last, after x has been read
        if (y0 == x) {
            st = enqueue_fake_quant(x, y1, cols, m, amax1, s);
            return st != NVFP4_OK ? st : enqueue_fake_quant(x, y0, cols, m, amax0, s);
        }
        st = enqueue_fake_quant(x, y0, cols, m, amax0, s);
        return st != NVFP4_OK ? st : enqueue_fake_quant(x, y1, cols, m, amax1, s);
    }
    const int64_t nh = 2 * m.nblocks;
    k_fake_quant_dual<false><<<persistent_grid(nh, (int64_t)kThreads * kUnroll, dual_wg_per_cu(nh)),
                               kThreads, 0, s>>>(static_cast<const uint4*>(x), static_cast<uint4*>(y0),
                                                 static_cast<uint4*>(y1), nh, AmaxIn{{amax0, amax1}});
    return launched();
}

nvfp4_status nvfp4_quantize_pack(const void* x, int64_t rows, int64_t cols,
                                 const float* amax_in, float* amax_out,
                                 uint8_t* packed, uint8_t* scales, float* global_scale,
                                 void* stream)
{
    Matrix m;
    nvfp4_status st = check_matrix(rows, cols, &m);
    if (st != NVFP4_OK)
        return st;
    const int64_t n = m.numel;
    if ((n > 0 && (!x || !packed || !scales)) || !global_scale || (!amax_in && !amax_out))
        return NVFP4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(packed, 8) || !aligned(global_scale, 4) ||
        (amax_in && !aligned(amax_in, 4)) || (!amax_in && !aligned(amax_out, 4)))
        return NVFP4_ERR_ALIGN;
    const uint64_t xb = 2 * (uint64_t)n, pb = 8 * (uint64_t)m.nblocks, sb = (uint64_t)m.nblocks;
    const void* outs[4] = {packed, scales, global_scale, amax_in ? nullptr : amax_out};
    const uint64_t lens[4] = {pb, sb, 4, amax_in ? 0u : 4u};
    for (int i = 0; i < 4; ++i) {
        if (overlap(outs[i], lens[i], x, xb) || (amax_in && overlap(outs[i], lens[i], amax_in, 4)))
            return NVFP4_ERR_OVERLAP;
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], lens[i], outs[j], lens[j]))
                return NVFP4_ERR_OVERLAP;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    const float* a = amax_in;
    if (!a) {
        st = enqueue_amax_one(x, n, amax_out, s, amax_alloc_bytes(2 * n, NVFP4_QP_AMAX_ALLOC_MID));
        if (st != NVFP4_OK)
            return st;
        a = amax_out;
    }
    return enqueue_quantize_pack(x, cols, m, packed, scales, global_scale, a, s);
}

nvfp4_status nvfp4_dequant_unpack(const uint8_t* packed, const uint8_t* scales,
                                  const float* global_scale, int64_t rows, int64_t cols,
                                  void* y, void* stream)
{
    Matrix m;
    nvfp4_status st = check_matrix(rows, cols, &m);
    if (st != NVFP4_OK)
        return st;
    if (m.numel == 0)
        return NVFP4_OK;
    if (!packed || !scales || !global_scale || !y)
        return NVFP4_ERR_NULL;
    if (!aligned(packed, 8) || !aligned(y, 16) || !aligned(global_scale, 4))
        return NVFP4_ERR_ALIGN;
    const uint64_t yb = 2 * (uint64_t)m.numel;
    if (overlap(y, yb, packed, 8 * (uint64_t)m.nblocks) || overlap(y, yb, scales, (uint64_t)m.nblocks) ||
        overlap(y, yb, global_scale, 4))
        return NVFP4_ERR_OVERLAP;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (half_rows(cols, m)) {
        const HalfRows g = half_rows_of(y, cols, m);
        const unsigned grid = persistent_grid(g.nhalves, (int64_t)kThreads * kDqUnroll, NVFP4_DQ_WG_PER_CU);
        const uint32_t* pv = reinterpret_cast<const uint32_t*>(packed);
        uint16_t* yh = static_cast<uint16_t*>(y);
        if (cols % 2 == 0)
            k_dequant_unpack_rows<false><<<grid, kThreads, 0, s>>>(pv, scales, global_scale, yh, g);
        else
            k_dequant_unpack_rows<true><<<grid, kThreads, 0, s>>>(pv, scales, global_scale, yh, g);
        return launched();
    }
    if (m.ragged) {
        const RaggedShape g{cols, m.nbr, m.nblocks};
        k_dequant_unpack_ragged<<<persistent_grid(m.nblocks, kThreads, kRaggedWgPerCu), kThreads, 0, s>>>(
            reinterpret_cast<const uint2*>(packed), scales, global_scale, static_cast<uint16_t*>(y), g);
        return launched();
    }
    k_dequant_unpack<<<persistent_grid(2 * m.nblocks, (int64_t)kThreads * kDqUnroll, NVFP4_DQ_WG_PER_CU), kThreads, 0, s>>>(
        reinterpret_cast<const uint32_t*>(packed), scales, global_scale, static_cast<uint4*>(y), 2 * m.nblocks);
    return launched();
}

nvfp4_status nvfp4_observer_update(float* state, const float* cur, int mode, float decay,
                                   void* stream)
{
    if (!state || !cur)
        return NVFP4_ERR_NULL;
    if (!aligned(state, 4) || !aligned(cur, 4))
        return NVFP4_ERR_ALIGN;
    if (!observer_args_ok(mode, decay))
        return NVFP4_ERR_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    k_observer<<<1, 1, 0, s>>>(cur, ObserverArgs{{state, nullptr}, {mode, 0}, {decay, 0.0f}}, 1);
    return launched();
}

nvfp4_status nvfp4_fake_quant_ws(const void* x, void* y, int64_t rows, int64_t cols, float* amax_out,
                                 void* workspace, void* stream)
{
    Matrix m;
    nvfp4_status st = check_fake_quant_ws(x, y, rows, cols, amax_out, &m);
    if (st != NVFP4_OK)
        return st;
    if (!workspace)
        return NVFP4_ERR_NULL;
    if (!aligned(workspace, 256))
        return NVFP4_ERR_ALIGN;
    const uint64_t bytes = 2 * (uint64_t)m.numel;
    const Region in[1] = {{x, bytes}};
    const Region out[3] = {{y, bytes}, {amax_out, amax_out ? 4u : 0u}, {workspace, NVFP4_WORKSPACE_BYTES}};
    if (check_regions(in, 1, out, 3, true) != NVFP4_OK)
        return NVFP4_ERR_OVERLAP;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    return enqueue_fake_quant_ws(x, y, cols, m, amax_out, workspace, s);
}

nvfp4_status nvfp4_fake_quant_noalloc(const void* x, void* y, int64_t rows, int64_t cols, float* amax_out,
                                      void* stream)
{
    Matrix m;
    nvfp4_status st = check_fake_quant_ws(x, y, rows, cols, amax_out, &m);
    if (st != NVFP4_OK)
        return st;
    const uint64_t bytes = 2 * (uint64_t)m.numel;
    const Region in[1] = {{x, bytes}};
    const Region out[2] = {{y, bytes}, {amax_out, amax_out ? 4u : 0u}};
    if (check_regions(in, 1, out, 2, true) != NVFP4_OK)
        return NVFP4_ERR_OVERLAP;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    void* ws = nullptr;
    if ((st = scratch_address(s, &ws)) != NVFP4_OK)
        return st;
    return enqueue_fake_quant_ws(x, y, cols, m, amax_out, ws, s);
}

nvfp4_status nvfp4_quantize_pack_ws(const void* x, int64_t rows, int64_t cols, float* amax_out,
                                    uint8_t* packed, uint8_t* scales, float* global_scale, void* workspace,
                                    void* stream)
{
    Matrix m;
    const nvfp4_status st = check_matrix(rows, cols, &m);
    if (st != NVFP4_OK)
        return st;
    if ((m.numel > 0 && (!x || !packed || !scales)) || !global_scale || !workspace)
        return NVFP4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(packed, 8) || !aligned(global_scale, 4) || !aligned(workspace, 256) ||
        (amax_out && !aligned(amax_out, 4)))
        return NVFP4_ERR_ALIGN;
    const Region in[1] = {{x, 2 * (uint64_t)m.numel}};
    const Region out[5] = {{packed, 8 * (uint64_t)m.nblocks},
                           {scales, (uint64_t)m.nblocks},
                           {global_scale, 4},
                           {amax_out, amax_out ? 4u : 0u},
                           {workspace, NVFP4_WORKSPACE_BYTES}};
    if (check_regions(in, 1, out, 5, false) != NVFP4_OK)
        return NVFP4_ERR_OVERLAP;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (!m.ragged || (m.numel > 0 && half_rows(cols, m))) {
        AmaxIn src;
        if (enqueue_amax_partials(&x, &m.numel, 1, workspace, s, &src, ObserverArgs{}, 0,
                                  amax_alloc_bytes(2 * m.numel, NVFP4_QP_AMAX_ALLOC_MID)) != NVFP4_OK)
            return NVFP4_ERR_HIP;
        src.store = amax_out;
        return enqueue_quantize_pack(x, cols, m, packed, scales, global_scale, src, s);
    }
    float* a = ws_amax(workspace, amax_out);
    if (enqueue_amax_ws(&x, &m.numel, 1, workspace, a, s) != NVFP4_OK)
        return NVFP4_ERR_HIP;
    return enqueue_quantize_pack(x, cols, m, packed, scales, global_scale, a, s);
}

nvfp4_status nvfp4_observe_fake_quant(const void* x, int64_t rows, int64_t cols, float* cur,
                                      float* state0, int mode0, float decay0, void* y0,
                                      float* state1, int mode1, float decay1, void* y1, void* workspace,
                                      void* stream)
{
    Matrix m;
    nvfp4_status st = check_matrix(rows, cols, &m);
    if (st != NVFP4_OK)
        return st;
    const bool two = state1 != nullptr;
    if (!cur || !state0 || !workspace || (m.numel > 0 && (!x || !y0 || (two && !y1))))
        return NVFP4_ERR_NULL;
    if ((!two && y1) || !observer_args_ok(mode0, decay0) || (two && !observer_args_ok(mode1, decay1)))
        return NVFP4_ERR_ARG;
    if (!aligned(x, 16) || !aligned(y0, 16) || !aligned(y1, 16) || !aligned(cur, 4) || !aligned(state0, 4) ||
        !aligned(state1, 4) || !aligned(workspace, 256))
        return NVFP4_ERR_ALIGN;
    const uint64_t bytes = 2 * (uint64_t)m.numel;
    const Region in[1] = {{x, bytes}};
    const Region out[6] = {{y0, y0 ? bytes : 0u}, {y1, y1 ? bytes : 0u}, {cur, 4}, {state0, 4},
                           {state1, two ? 4u : 0u}, {workspace, NVFP4_WORKSPACE_BYTES}};
    if (check_regions(in, 1, out, 6, true) != NVFP4_OK)
        return NVFP4_ERR_OVERLAP;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    const ObserverArgs obs{{state0, state1}, {mode0, mode1}, {decay0, decay1}};
    const int64_t nh = 2 * m.nblocks;
    const int wg_per_cu = two ? dual_wg_per_cu(nh)
                              : quant_wg_per_cu(nh, NVFP4_FQ_MID_WG_PER_CU, NVFP4_FQ_WG_PER_CU);
    const unsigned grid = persistent_grid(nh, (int64_t)kThreads * kUnroll, wg_per_cu);
    if (m.numel > 0 && !m.ragged) {
        // the amax pass (which also copies the states), then one pass that reduces
        // the partials into *cur, steps the observers and fake-quantizes with the
        // new states
        AmaxIn src;
        if (enqueue_amax_partials(&x, &m.numel, 1, workspace, s, &src, obs, two ? 2 : 1,
                                  amax_alloc_bytes(2 * m.numel, NVFP4_FQ_AMAX_ALLOC_MID)) != NVFP4_OK)
            return NVFP4_ERR_HIP;
        src.store = cur;
        if (!two)
            return enqueue_fake_quant(x, y0, cols, m, src, s);
        k_fake_quant_dual<true><<<grid, kThreads, 0, s>>>(static_cast<const uint4*>(x), static_cast<uint4*>(y0),
                                                          static_cast<uint4*>(y1), nh, src);
        return launched();
    }
    // the amax pass, then one workgroup reduces its partial maxima into *cur and
    // steps both observers on it
    if (enqueue_amax_ws(&x, &m.numel, 1, workspace, cur, s, obs, two ? 2 : 1) != NVFP4_OK)
        return NVFP4_ERR_HIP;
    if (m.numel == 0)
        return NVFP4_OK;
    if (!two)
        return enqueue_fake_quant(x, y0, cols, m, state0, s);
    if (m.ragged) {
        // two passes; an output written in place goes last, after x has been read
        const bool swap = y0 == x;
        st = enqueue_fake_quant(x, swap ? y1 : y0, cols, m, swap ? state1 : state0, s);
        return st != NVFP4_OK ? st : enqueue_fake_quant(x, swap ? y0 : y1, cols, m, swap ? state0 : state1, s);
    }
    k_fake_quant_dual<false><<<grid, kThreads, 0, s>>>(static_cast<const uint4*>(x), static_cast<uint4*>(y0),
                                                       static_cast<uint4*>(y1), nh, AmaxIn{{state0, state1}});
    return launched();
}

nvfp4_status nvfp4_linear(const void* x, int64_t m, int64_t k, const uint8_t* packed,
                          const uint8_t* scales, const float* global_scale, int64_t n, const void* bias,
                          void* y, void* stream)
{
    if (m < 0 || n < 0 || k < 32 || k % 32 != 0)
        return NVFP4_ERR_SHAPE;
    if (k > ((int64_t)1 << 40) || m > ((int64_t)1 << 40) / k || n > ((int64_t)1 << 40) / k ||
        (m > 0 && n > ((int64_t)1 << 50) / m) || (m + 63) / 64 > 65535)
        return NVFP4_ERR_SHAPE;
    if (!packed || !scales || !global_scale || (m > 0 && (!x || !y)))
        return NVFP4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(scales, 2) || !aligned(global_scale, 4) ||
        !aligned(bias, 2) || !aligned(y, 2))
        return NVFP4_ERR_ALIGN;
    const uint64_t yb = 2 * (uint64_t)(m * n);
    if (overlap(y, yb, x, 2 * (uint64_t)(m * k)) || overlap(y, yb, packed, (uint64_t)(n * k / 2)) ||
        overlap(y, yb, scales, (uint64_t)(n * k / 16)) || overlap(y, yb, global_scale, 4) ||
        overlap(y, yb, bias, bias ? 2 * (uint64_t)n : 0))
        return NVFP4_ERR_OVERLAP;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (m == 0 || n == 0)
        return NVFP4_OK;
    if (m <= 16)
        return enqueue_linear_mt<1>(x, m, k, packed, scales, global_scale, n, bias, y, s);
    if (m <= 32)
        return enqueue_linear_mt<2>(x, m, k, packed, scales, global_scale, n, bias, y, s);
    // the LDS-staged kernel keeps a tile's 256 rows of x below 2^31 bytes (32-bit buffer offsets)
    const bool lds_k = k % kLdsK == 0 && k < ((int64_t)1 << 22);
    const int64_t cus = linear_cus();
    if (lds_k && NVFP4_LIN_NARROW && m > 128 && m <= 256 && 2 * ((n + 127) / 128) > cus && (n + 127) / 128 <= cus)
        // 129-256 rows, whose 128 x 128 tiles would not fit one per CU: one round of 256 x 128 tiles
        return enqueue_linear_lds<8, 4, 2, 2>(x, m, k, packed, scales, global_scale, 0, n, n, bias, y, s);
    if (lds_k && m >= NVFP4_LIN_LDS_M && (n + 255) / 256 <= 65535)
        return enqueue_linear_lds_large(x, m, k, packed, scales, global_scale, n, bias, y, s);
    if (lds_k && m >= NVFP4_LIN_LDS_SMALL_M && (n + 127) / 128 <= 65535)
        // Two K groups (8 waves, twice the LDS) while the tiles fit one per CU; with
        // more tiles two single-group workgroups share a CU instead.
        return NVFP4_LIN_LDS_KG2 && (k / kLdsK) % 2 == 0 && ((m + 127) / 128) * ((n + 127) / 128) <= compute_units()
                   ? enqueue_linear_lds<4, 2, 2, 2, 2>(x, m, k, packed, scales, global_scale, 0, n, n, bias, y, s)
                   : enqueue_linear_lds<4, 2, 2, 2>(x, m, k, packed, scales, global_scale, 0, n, n, bias, y, s);
    constexpr int kNW = NVFP4_TILE_NW;
    if (m < NVFP4_LIN_TILED_M || (n + 32 * kNW * kTileWaves - 1) / (32 * kNW * kTileWaves) > 65535)
        return enqueue_linear_mt<4>(x, m, k, packed, scales, global_scale, n, bias, y, s);
    if (m <= NVFP4_TILE_SMALL_M)
        return enqueue_linear_tiled<NVFP4_TILE_MW_SMALL, kNW>(x, m, k, packed, scales, global_scale, n, bias, y, s);
    return enqueue_linear_tiled<NVFP4_TILE_MW, kNW>(x, m, k, packed, scales, global_scale, n, bias, y, s);
}

// MXFP4 ragged rows take the quarter-block kernels while the quarter count fits
// their 32-bit index (the same bound as the NVFP4 half-block kernels'), and the
// one-lane-per-block kernels beyond.
bool mx_rows(const Matrix& m)
{
    return m.ragged && 4 * m.nblocks < 2 * (int64_t)NVFP4_HALF_ROWS_MAX_BLOCKS;
}

HalfRows mx_rows_of(const void* x, int64_t cols, const Matrix& m)
{
    return HalfRows{static_cast<const uint16_t*>(x), cols, (uint32_t)(4 * m.nbr), 4 * m.nblocks};
}

nvfp4_status nvfp4_mx_fake_quant(const void* x, void* y, int64_t rows, int64_t cols, void* stream)
{
    Matrix m;
    const nvfp4_status st = check_mx_matrix(rows, cols, &m);
    if (st != NVFP4_OK)
        return st;
    if (m.numel > 0 && (!x || !y))
        return NVFP4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(y, 16))
        return NVFP4_ERR_ALIGN;
    const uint64_t bytes = 2 * (uint64_t)m.numel;
    if (x != y && overlap(x, bytes, y, bytes))
        return NVFP4_ERR_OVERLAP;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (m.numel == 0)
        return NVFP4_OK;
    if (mx_rows(m)) {
        const HalfRows g = mx_rows_of(x, cols, m);
        const unsigned grid = persistent_grid(g.nhalves, (int64_t)kThreads * kUnroll, NVFP4_MX_WG_PER_CU);
        if (cols % 2 == 0)
            k_mx_fake_quant_rows<false><<<grid, kThreads, 0, s>>>(g, static_cast<uint16_t*>(y));
        else
            k_mx_fake_quant_rows<true><<<grid, kThreads, 0, s>>>(g, static_cast<uint16_t*>(y));
        return launched();
    }
    if (m.ragged) {
        k_mx_fake_quant_ragged<<<persistent_grid(m.nblocks, kThreads, kRaggedWgPerCu), kThreads, 0, s>>>(
            static_cast<const uint16_t*>(x), static_cast<uint16_t*>(y), RaggedShape{cols, m.nbr, m.nblocks});
        return launched();
    }
    const int64_t nq = 4 * m.nblocks;
    k_mx_fake_quant<<<persistent_grid(nq, (int64_t)kThreads * kUnroll, NVFP4_MX_WG_PER_CU), kThreads, 0, s>>>(
        static_cast<const uint4*>(x), static_cast<uint4*>(y), nq);
    return launched();
}

nvfp4_status nvfp4_mx_quantize_pack(const void* x, int64_t rows, int64_t cols, uint8_t* packed, float* scales,
                                    void* stream)
{
    Matrix m;
    const nvfp4_status st = check_mx_matrix(rows, cols, &m);
    if (st != NVFP4_OK)
        return st;
    if (m.numel > 0 && (!x || !packed || !scales))
        return NVFP4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(scales, 4))
        return NVFP4_ERR_ALIGN;
    const Region in[1] = {{x, 2 * (uint64_t)m.numel}};
    const Region out[2] = {{packed, 16 * (uint64_t)m.nblocks}, {scales, 4 * (uint64_t)m.nblocks}};
    if (check_regions(in, 1, out, 2, false) != NVFP4_OK)
        return NVFP4_ERR_OVERLAP;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (m.numel == 0)
        return NVFP4_OK;
    if (mx_rows(m)) {
        const HalfRows g = mx_rows_of(x, cols, m);
        const unsigned grid = persistent_grid(g.nhalves, (int64_t)kThreads * kUnroll, NVFP4_MX_WG_PER_CU);
        uint32_t* pv = reinterpret_cast<uint32_t*>(packed);
        if (cols % 2 == 0)
            k_mx_quantize_pack_rows<false><<<grid, kThreads, 0, s>>>(g, pv, scales);
        else
            k_mx_quantize_pack_rows<true><<<grid, kThreads, 0, s>>>(g, pv, scales);
        return launched();
    }
    if (m.ragged) {
        k_mx_quantize_pack_ragged<<<persistent_grid(m.nblocks, kThreads, kRaggedWgPerCu), kThreads, 0, s>>>(
            static_cast<const uint16_t*>(x), reinterpret_cast<uint4*>(packed), scales,
            RaggedShape{cols, m.nbr, m.nblocks});
        return launched();
    }
    const int64_t nq = 4 * m.nblocks;
    k_mx_quantize_pack<<<persistent_grid(nq, (int64_t)kThreads * kUnroll, NVFP4_MX_WG_PER_CU), kThreads, 0, s>>>(
        static_cast<const uint4*>(x), reinterpret_cast<uint32_t*>(packed), scales, nq);
    return launched();
}

nvfp4_status nvfp4_mx_dequant_unpack(const uint8_t* packed, const float* scales, int64_t rows, int64_t cols,
                                     void* y, void* stream)
{
    Matrix m;
    const nvfp4_status st = check_mx_matrix(rows, cols, &m);
    if (st != NVFP4_OK)
        return st;
    if (m.numel == 0)
        return NVFP4_OK;
    if (!packed || !scales || !y)
        return NVFP4_ERR_NULL;
    if (!aligned(packed, 16) || !aligned(scales, 4) || !aligned(y, 16))
        return NVFP4_ERR_ALIGN;
    const Region in[2] = {{packed, 16 * (uint64_t)m.nblocks}, {scales, 4 * (uint64_t)m.nblocks}};
    const Region out[1] = {{y, 2 * (uint64_t)m.numel}};
    if (check_regions(in, 2, out, 1, false) != NVFP4_OK)
        return NVFP4_ERR_OVERLAP;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (mx_rows(m)) {
        const HalfRows g = mx_rows_of(y, cols, m);
        const unsigned grid = persistent_grid(g.nhalves, (int64_t)kThreads * kDqUnroll, NVFP4_MX_WG_PER_CU);
        const uint32_t* pv = reinterpret_cast<const uint32_t*>(packed);
        if (cols % 2 == 0)
            k_mx_dequant_unpack_rows<false><<<grid, kThreads, 0, s>>>(pv, scales, static_cast<uint16_t*>(y), g);
        else
            k_mx_dequant_unpack_rows<true><<<grid, kThreads, 0, s>>>(pv, scales, static_cast<uint16_t*>(y), g);
        return launched();
    }
    if (m.ragged) {
        k_mx_dequant_unpack_ragged<<<persistent_grid(m.nblocks, kThreads, kRaggedWgPerCu), kThreads, 0, s>>>(
            reinterpret_cast<const uint4*>(packed), scales, static_cast<uint16_t*>(y),
            RaggedShape{cols, m.nbr, m.nblocks});
        return launched();
    }
    const int64_t nq = 4 * m.nblocks;
    k_mx_dequant_unpack<<<persistent_grid(nq, (int64_t)kThreads * kDqUnroll, NVFP4_MX_WG_PER_CU), kThreads, 0,
                          s>>>(reinterpret_cast<const uint32_t*>(packed), scales, static_cast<uint4*>(y), nq);
    return launched();
}

}  // extern "C"
