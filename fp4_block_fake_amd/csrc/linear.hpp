// The linear layer over a packed NVFP4 weight: bf16 MFMA with the weight decoded
// in registers (included by nvfp4.hip).

#ifndef NVFP4_LINEAR_HPP
#define NVFP4_LINEAR_HPP

#include <type_traits>
#include <utility>

#include "device.hpp"

namespace {

// ---------------------------------------------------------------- linear over a packed weight
//
// y[m, n] = bf16( sum_k x[m, k] * w[n, k] + b[n] ), w = the bf16 weight that
// dequant-unpack would write (VideoX-Fun page, the per-forward reconstruction:
// the packed weight is dequantized to bf16 and the layer's linear runs on it).
// Here the dequantization happens in registers, straight into the B operand of
// bf16 MFMAs, so the bf16 weight never exists in memory: the weight costs 0.5625
// bytes per element of HBM traffic instead of 2 (read) + 2 (write) + 2 (read).
//
// v_mfma_f32_16x16x32_bf16 operand layout (checked on MI355X): lane l holds
// A[l % 16][8 (l / 16) .. + 8], B[8 (l / 16) .. + 8][l % 16], and accumulator
// element i of lane l is D[4 (l / 16) + i][l % 16].  The sum over k may visit k
// in any order, so in a KS-wide step lane group g = l / 16 takes the KS / 4
// contiguous k from KS g / 4 for all KS / 32 MFMAs of the step (MFMA q uses the
// q-th 8 of them), for A and B alike: per weight row, KS / 128 16-byte loads of
// codes and one load of their KS / 64 scale bytes; per x row, KS / 32 16-byte
// loads.
//
// A workgroup computes a tile of 16 MT rows of x by 16 NT rows of w; its W
// waves split K (steps interleaved) and their partial sums meet in LDS, added in
// wave order, so results do not depend on timing.  Rows past the end of x or w
// read row 0 instead: accumulator element D[m][n] depends only on row m of x
// and row n of w, and those rows are never stored, so every load stays
// unconditional (no branch splits the load pipeline).
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kLinDepth = NVFP4_LIN_DEPTH;
constexpr size_t kLinLdsBudget = 64 * 1024 - 128 * sizeof(float);   // beside the sd table

// 16-row tiles of x whose partial sums waves 1..W-1 of k_linear hand over per
// round: all MT when they fit in kLinLdsBudget, else one per round.
template <int MT, int NT, int W>
constexpr int lin_partial_tiles()
{
    return (size_t)(W - 1) * MT * NT * 64 * sizeof(f32x4) <= kLinLdsBudget ? MT : 1;
}

// Eight codes (one dword) -> the B operand: their bf16 values decode * sd, as
// dequant-unpack writes them.
__device__ __forceinline__ bf16x8 decode_operand(uint32_t c, float sd)
{
    return __builtin_bit_cast(bf16x8, decode_half(c, sd));
}

__device__ __forceinline__ uint32_t dword_of(const uint4& v, int i)
{
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Dynamic LDS of the linear kernel: with SL, the scale rows of the workgroup's
// weight tiles during the K loop; then the partial sums of waves 1..W-1.
extern __shared__ __align__(16) uint8_t lin_lds[];

template <int MT, int NT, int W, int KS, bool SL>
__global__ __launch_bounds__(64 * W) void k_linear(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                     const uint32_t* __restrict__ packed,
                                                     const uint8_t* __restrict__ scales,
                                                     const float* __restrict__ gs_in, int64_t N,
                                                     const uint16_t* __restrict__ bias,
                                                     uint16_t* __restrict__ y)
{
    static_assert(KS == 128 || KS == 256, "step width");
    constexpr int kQ = KS / 32;            // MFMAs per weight tile and step
    constexpr int kCv = KS / 128;          // 16-byte code loads per row and step
    __shared__ float sd_of[128];
    const float gs = *gs_in;
    if (threadIdx.x < 128)
        sd_of[threadIdx.x] = e4m3_decode(threadIdx.x) / gs;

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16 * NT, m0 = (int64_t)blockIdx.y * 16 * MT;
    const int64_t cw = K / 8, sw = K / 16;           // code dwords and scale bytes per weight row
    const bool scale_dword = KS == 256 && (sw & 3) == 0 && (SL || ((uintptr_t)scales & 3) == 0);
    if (SL) {
        // The workgroup's scale rows are contiguous: one coalesced copy into LDS
        // (16-byte pieces when aligned, 2-byte otherwise; every row is an even
        // number of bytes).
        const int64_t rows = N - n0 < 16 * NT ? N - n0 : 16 * NT;
        const uint8_t* src = scales + n0 * sw;
        const int64_t bytes = rows * sw;
        if (((uintptr_t)src & 15) == 0) {
            for (int64_t i = threadIdx.x; i < bytes / 16; i += 64 * W)
                reinterpret_cast<uint4*>(lin_lds)[i] = reinterpret_cast<const uint4*>(src)[i];
            for (int64_t i = bytes / 16 * 16 + 2 * threadIdx.x; i < bytes; i += 2 * 64 * W)
                *reinterpret_cast<uint16_t*>(lin_lds + i) = *reinterpret_cast<const uint16_t*>(src + i);
        } else {
            for (int64_t i = 2 * threadIdx.x; i < bytes; i += 2 * 64 * W)
                *reinterpret_cast<uint16_t*>(lin_lds + i) = *reinterpret_cast<const uint16_t*>(src + i);
        }
    }
    __syncthreads();

    const uint32_t* wrow[NT];
    const uint8_t* srow[NT];               // without SL: the scale row in HBM
    uint32_t soff[NT];                     // with SL: the scale row's offset in LDS
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int64_t n = n0 + 16 * t + r;
        wrow[t] = packed + (n < N ? n : 0) * cw;
        srow[t] = scales + (n < N ? n : 0) * sw;
        soff[t] = (uint32_t)((n < N ? 16 * t + r : 0) * sw);
    }
    // scale bytes [k / 16, k / 16 + bytes) of weight tile t (bytes = 1, 2 or 4)
    auto scale_bytes = [&](int t, int64_t k, int bytes) -> uint32_t {
        if (SL) {
            const uint8_t* sp = lin_lds + soff[t] + k / 16;
            if (bytes == 1)
                return *sp;
            if (bytes == 2 || !scale_dword)
                return bytes == 2 ? *reinterpret_cast<const uint16_t*>(sp)
                                  : (uint32_t)*reinterpret_cast<const uint16_t*>(sp) |
                                    ((uint32_t)*reinterpret_cast<const uint16_t*>(sp + 2) << 16);
            return *reinterpret_cast<const uint32_t*>(sp);
        }
        const uint8_t* sp = srow[t] + k / 16;
        if (bytes == 1)
            return *sp;
        if (bytes == 2)
            return *reinterpret_cast<const uint16_t*>(sp);
        if (scale_dword)
            return *reinterpret_cast<const uint32_t*>(sp);
        return (uint32_t)*reinterpret_cast<const uint16_t*>(sp) |
               ((uint32_t)*reinterpret_cast<const uint16_t*>(sp + 2) << 16);
    };
    const uint16_t* xrow[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int64_t m = m0 + 16 * i + r;
        xrow[i] = x + (m < M ? m : 0) * K;
    }

    f32x4 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int t = 0; t < NT; ++t)
            acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // The weight operands of a step (codes and scale bytes, the HBM stream) are
    // loaded kLinDepth steps ahead; x (from L2) one step ahead.
    struct WOp {
        uint4 c[NT][kCv];
        uint32_t sc[NT];                   // KS / 64 scale bytes, lowest first
    };
    struct XOp {
        uint4 a[MT][kQ];
    };
    auto load_w = [&](int64_t st, WOp& o) {
        const int64_t k0 = st * KS + (KS / 4) * g;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int v = 0; v < kCv; ++v)
                o.c[t][v] = *reinterpret_cast<const uint4*>(wrow[t] + k0 / 8 + 4 * v);
            o.sc[t] = scale_bytes(t, k0, KS / 64);
        }
    };
    auto load_x = [&](int64_t st, XOp& o) {
        const int64_t k0 = st * KS + (KS / 4) * g;
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int q = 0; q < kQ; ++q)
                o.a[i][q] = *reinterpret_cast<const uint4*>(xrow[i] + k0 + 8 * q);
    };
    auto mma_step = [&](const WOp& o, const XOp& xo) {
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const float sd = sd_of[(o.sc[t] >> (8 * (q / 2))) & 0x7Fu];
                const bf16x8 b = decode_operand(dword_of(o.c[t][q / 4], q % 4), sd);
#pragma unroll
                for (int i = 0; i < MT; ++i)
                    acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xo.a[i][q]), b,
                                                                        acc[i][t], 0, 0, 0);
            }
        }
    };
    // A wave's j-th step uses ring[j % D] and xbuf[j % 2]; D is even, so both
    // indices are compile-time constants in the unrolled body.
    static_assert(kLinDepth % 2 == 0, "the x double buffer alternates with the ring");
    const int64_t steps = K / KS;
    WOp ring[kLinDepth];
    XOp xbuf[2];
#pragma unroll
    for (int d = 0; d < kLinDepth; ++d)
        if (wave + d * W < steps)
            load_w(wave + d * W, ring[d]);
    if (wave < steps)
        load_x(wave, xbuf[0]);
    for (int64_t st = wave; st < steps; st += kLinDepth * W) {
#pragma unroll
        for (int d = 0; d < kLinDepth; ++d) {
            const int64_t at = st + d * W;
            if (at < steps) {
                if (at + W < steps)
                    load_x(at + W, xbuf[(d + 1) % 2]);
                mma_step(ring[d], xbuf[d % 2]);
                if (at + kLinDepth * W < steps)
                    load_w(at + kLinDepth * W, ring[d]);
            }
        }
    }
    // K % KS: 32-wide steps shared out over the waves, in the plain layout
    // (lane group g takes k in [8 g, 8 g + 8) of the step)
    for (int64_t kt = steps * KS + 32 * wave; kt < K; kt += 32 * W) {
        const int64_t k0 = kt + 8 * g;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const bf16x8 b = decode_operand(wrow[t][k0 / 8], sd_of[scale_bytes(t, k0, 1) & 0x7Fu]);
#pragma unroll
            for (int i = 0; i < MT; ++i) {
                const uint4 a = *reinterpret_cast<const uint4*>(xrow[i] + k0);
                acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), b, acc[i][t],
                                                                    0, 0, 0);
            }
        }
    }

    // waves 1..W-1 hand their partial sums to wave 0, which adds them in order
    // (through the LDS the scales used, once every wave is past the K loop); when
    // they do not all fit at once, one 16-row tile of x per round
    constexpr int kPer = lin_partial_tiles<MT, NT, W>();
    static_assert((size_t)(W - 1) * kPer * NT * 64 * sizeof(f32x4) <= kLinLdsBudget, "one round fits in LDS");
    f32x4 (*partial)[kPer * NT][64] = reinterpret_cast<f32x4 (*)[kPer * NT][64]>(lin_lds);
#pragma unroll
    for (int rd = 0; rd < MT / kPer; ++rd) {
        if (SL || rd > 0)
            __syncthreads();
        if (wave > 0) {
#pragma unroll
            for (int i = 0; i < kPer; ++i)
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    partial[wave - 1][i * NT + t][lane] = acc[rd * kPer + i][t];
        }
        __syncthreads();
        if (wave != 0)
            continue;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int ti = rd * kPer + i;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                f32x4 v = acc[ti][t];
#pragma unroll
                for (int w = 0; w < W - 1; ++w)
                    v += partial[w][i * NT + t][lane];
                const int64_t n = n0 + 16 * t + r;
                if (n >= N)
                    continue;
                const float b = bias ? bf16_value(bias[n]) : 0.0f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t m = m0 + 16 * ti + 4 * g + e;
                    if (m < M) {
                        const f32x2 o = {v[e] + b, 0.0f};
                        y[m * N + n] =
                            (uint16_t)(__builtin_bit_cast(uint32_t, __builtin_convertvector(o, bf16x2)) & 0xFFFFu);
                    }
                }
            }
        }
    }
}

// The linear layer for many rows of x.  A workgroup covers 32 MW rows of x and
// 32 NW kTileWaves weight rows.  The x tile of each K step goes through LDS
// (double-buffered: the next step's tile is loaded while this one is used) and
// is shared by the kTileWaves waves; each wave owns NW tiles of 32 weight rows
// and decodes their codes straight into its B operands, so every weight is
// decoded once per workgroup and used by MW MFMA tiles.  The waves split N, so
// there are no partial sums to combine.  The tiles are 32 x 32 x 16 MFMAs, which
// do twice the FLOPs per operand byte of 16 x 16 x 32 ones (half the LDS reads
// of x per FLOP; measured 1.25x faster here).  Operand layouts (checked on
// MI355X): lane l holds A[l % 32][8 (l / 32) .. +8] and B[8 (l / 32) .. +8][l % 32];
// accumulator j of lane l is D[(j % 4) + 8 (j / 4) + 4 (l / 32)][l % 32].  Within a
// K step, lane half h takes K indices [KS/2 h, KS/2 (h + 1)) in MFMA slices of 8,
// for x and weights alike.
constexpr int kTileWaves = NVFP4_TILE_WAVES;
constexpr int kTileDepth = NVFP4_TILE_DEPTH;
static_assert(kTileDepth % 2 == 0, "the x double buffer alternates with the weight ring");
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int MW, int NW, int KS>
__global__ __launch_bounds__(64 * kTileWaves) void k_linear_tiled(const uint16_t* __restrict__ x, int64_t M,
                                                                    int64_t K, const uint8_t* __restrict__ packed,
                                                                    const uint8_t* __restrict__ scales,
                                                                    const float* __restrict__ gs_in, int64_t N,
                                                                    const uint16_t* __restrict__ bias,
                                                                    uint16_t* __restrict__ y)
{
    static_assert(KS == 32 || KS == 64, "step width");
    constexpr int kQ = KS / 16;                      // MFMA slices per step (and code dwords per lane)
    constexpr int kRows = 32 * MW;
    constexpr int kStride = KS + 8;
    constexpr int kPieces = kRows * KS / 8;
    constexpr int kPer = (kPieces + 64 * kTileWaves - 1) / (64 * kTileWaves);
    __shared__ float sd_of[128];
    uint16_t* xt = reinterpret_cast<uint16_t*>(lin_lds);     // [2][kRows][kStride]

    const float gs = *gs_in;
    if (threadIdx.x < 128)
        sd_of[threadIdx.x] = e4m3_decode(threadIdx.x) / gs;

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int c = lane & 31, h = lane >> 5;
    // Workgroups go to the 8 XCDs round-robin by id.  With the remap, XCD k gets a
    // contiguous run of weight tiles with all their x tiles, so a weight tile's codes
    // are fetched into one XCD's L2 and reused there by its other x tiles.  Measured
    // on the c5 weight: M = 128 162 -> 136 us, 256 210 -> 188, 1024 634 -> 597; at
    // M = 2048 (16 x tiles) it was slower (1122 -> 1177 us), so up to 8 x tiles only.
    uint32_t bx = blockIdx.x, by = blockIdx.y;
    if (NVFP4_TILE_XCD_REMAP && gridDim.x <= 8) {
        const uint32_t g = gridDim.x * gridDim.y, w = blockIdx.x + blockIdx.y * gridDim.x;
        if (g % 8 == 0) {
            const uint32_t l = (w % 8) * (g / 8) + w / 8;
            bx = l % gridDim.x;
            by = l / gridDim.x;
        }
    }
    const int64_t m0 = (int64_t)bx * kRows;
    const int64_t n0 = ((int64_t)by * kTileWaves + wave) * 32 * NW;
    const int64_t cb = K / 2, sb = K / 16;
    const uint8_t* wrow[NW];
    const uint8_t* srow[NW];
#pragma unroll
    for (int t = 0; t < NW; ++t) {
        const int64_t n = n0 + 32 * t + c;
        wrow[t] = packed + (n < N ? n : 0) * cb;
        srow[t] = scales + (n < N ? n : 0) * sb;
    }

    auto load_x = [&](int64_t st, uint4 (&v)[kPer]) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int p = threadIdx.x + 64 * kTileWaves * j;
            const int64_t m = m0 + p / (KS / 8);
            v[j] = p < kPieces && m < M
                       ? *reinterpret_cast<const uint4*>(x + m * K + st * KS + 8 * (p % (KS / 8)))
                       : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto store_x = [&](int buf, const uint4 (&v)[kPer]) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int p = threadIdx.x + 64 * kTileWaves * j;
            if (p < kPieces)
                *reinterpret_cast<uint4*>(xt + (buf * kRows + p / (KS / 8)) * kStride + 8 * (p % (KS / 8))) = v[j];
        }
    };
    // the lane's KS / 2 codes (kQ dwords) and their KS / 32 scale bytes, per weight tile
    auto load_w = [&](int64_t st, uint32_t (&cw)[NW][kQ], uint32_t (&sc)[NW]) {
        const int64_t k0 = st * KS + (KS / 2) * h;
#pragma unroll
        for (int t = 0; t < NW; ++t) {
            if (KS == 64) {
                const uint4 v = *reinterpret_cast<const uint4*>(wrow[t] + k0 / 2);
                cw[t][0] = v.x;
                cw[t][1] = v.y;
                cw[t][kQ - 2] = v.z;
                cw[t][kQ - 1] = v.w;
                sc[t] = *reinterpret_cast<const uint16_t*>(srow[t] + k0 / 16);
            } else {
                const uint2 v = *reinterpret_cast<const uint2*>(wrow[t] + k0 / 2);
                cw[t][0] = v.x;
                cw[t][kQ - 1] = v.y;
                sc[t] = srow[t][k0 / 16];
            }
        }
    };

    f32x16 acc[MW][NW];
#pragma unroll
    for (int i = 0; i < MW; ++i)
#pragma unroll
        for (int t = 0; t < NW; ++t)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                acc[i][t][j] = 0.0f;
    auto mma_step = [&](int buf, const uint32_t (&cw)[NW][kQ], const uint32_t (&sc)[NW]) {
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
            bf16x8 b[NW];
#pragma unroll
            for (int t = 0; t < NW; ++t)
                b[t] = decode_operand(cw[t][q], sd_of[(sc[t] >> (8 * (q / 2))) & 0x7Fu]);
#pragma unroll
            for (int i = 0; i < MW; ++i) {
                const uint4 a = *reinterpret_cast<const uint4*>(xt + (buf * kRows + 32 * i + c) * kStride +
                                                                (KS / 2) * h + 8 * q);
#pragma unroll
                for (int t = 0; t < NW; ++t)
                    acc[i][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), b[t],
                                                                        acc[i][t], 0, 0, 0);
            }
        }
    };

    const int64_t steps = K / KS;
    uint4 xv[kPer];
    uint32_t wc[kTileDepth][NW][kQ], wsb[kTileDepth][NW];
#pragma unroll
    for (int d = 0; d < kTileDepth; ++d)
        if (d < steps)
            load_w(d, wc[d], wsb[d]);
    load_x(0, xv);
    store_x(0, xv);
    __syncthreads();
    for (int64_t st0 = 0; st0 < steps; st0 += kTileDepth) {
#pragma unroll
        for (int d = 0; d < kTileDepth; ++d) {
            const int64_t st = st0 + d;
            if (st < steps) {
                const bool more = st + 1 < steps;
                if (more)
                    load_x(st + 1, xv);
                mma_step(d & 1, wc[d], wsb[d]);
                if (st + kTileDepth < steps)
                    load_w(st + kTileDepth, wc[d], wsb[d]);
                if (more)
                    store_x((d & 1) ^ 1, xv);
                __syncthreads();
            }
        }
    }

#pragma unroll
    for (int i = 0; i < MW; ++i) {
#pragma unroll
        for (int t = 0; t < NW; ++t) {
            const int64_t n = n0 + 32 * t + c;
            if (n >= N)
                continue;
            const float b = bias ? bf16_value(bias[n]) : 0.0f;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int64_t m = m0 + 32 * i + (j % 4) + 8 * (j / 4) + 4 * h;
                if (m < M) {
                    const f32x2 o = {acc[i][t][j] + b, 0.0f};
                    y[m * N + n] = (uint16_t)(__builtin_bit_cast(uint32_t, __builtin_convertvector(o, bf16x2)) & 0xFFFFu);
                }
            }
        }
    }
}

// ---------------------------------------------------------------- linear, weight tiles decoded into LDS
//
// For many rows of x (the layer is compute-bound there), the weight is decoded
// once per workgroup and K step into LDS as bf16, and both MFMA operands are read
// from LDS, so each weight element is decoded once per BM rows of x instead of
// once per 32-row x tile of a wave.  A workgroup of W waves computes a tile of
// BM = 32 TM WM rows of x by BN = 32 TN W / WM weight rows; wave w owns x rows
// 32 TM (w % WM) .. + 32 TM against weight rows 32 TN (w / WM) .. + 32 TN (TM x TN
// tiles of v_mfma_f32_32x32x16_bf16, operand and accumulator layouts as in
// k_linear_tiled).  Per 64-wide K step, each thread stages BM / (8 W) 16-byte
// pieces of x and decodes the 32 weight codes (16 bytes, two block scales) of
// one half row into 64 bytes of bf16: the same decode as dequant-unpack, so the
// weight is bit for bit the tensor dequant-unpack writes.  LDS holds two stages
// of both tiles (the next stage is written while this one is read); x loads run
// two steps ahead in registers, code loads four.  The next stage's decode and
// LDS writes sit between this stage's MFMA slices so that the VALU work overlaps
// the matrix cores.  Rows of x past M read row M - 1 and weight rows past N read
// row N - 1; neither is stored (an output element depends only on its own rows).
// Shapes used: 8 waves, 256 x 256 (WM 4, TM 2, TN 4: two waves per SIMD at 240
// VGPRs), and 4 waves, 128 x 128 (WM 2, TM 2, TN 2) for fewer rows of x, where
// the large tile would leave CUs idle; that one in two K groups (8 waves) when
// its tiles fit one per CU, which otherwise would hold one wave per SIMD.  A
// narrower tile (TN < 4, 64 TN weight rows per workgroup) leaves the weight
// staging to the first 2 kN threads (whole waves); it serves the last, partial
// round of 256 x 256 tiles, re-tiled so that one round of narrower tiles covers
// it.  y has row stride ldy, so a launch can cover a range of weight rows
// (packed, scales, bias and y offset by the caller).
constexpr int kLdsK = 64;
constexpr int kLdsStride = kLdsK + 8;          // bf16 per LDS row (padding against bank conflicts)
constexpr int kLdsXDepth = 2;                  // register stages of x loads in flight

// A raw buffer resource over [base, base + bytes) (bytes < 2^31), built from
// values every lane holds alike and kept in scalar registers (readfirstlane), so
// that loads through it need no per-lane descriptor.  Reads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_resource(const void* base, int64_t bytes)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const int n = __builtin_amdgcn_readfirstlane((int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0, n,
                                             0x00020000);
}

// f(integral_constant<int, I>) for I = 0 .. sizeof...(I) - 1, in order.
template <typename F, std::size_t... I>
__device__ __forceinline__ void for_each_index(F&& f, std::index_sequence<I...>)
{
    (f(std::integral_constant<int, (int)I>{}), ...);
}

template <int W, int WM, int TM, int TN>
struct LdsTile {
    static constexpr int kWN = W / WM;                     // waves along the weight rows
    static constexpr int kM = 32 * TM * WM;                // rows of x per workgroup
    static constexpr int kN = 32 * TN * kWN;               // weight rows per workgroup
    static constexpr int kT = 64 * W;                      // threads
    static constexpr int kXP = kM * (kLdsK / 8) / kT;      // 16-byte pieces of x per thread and step
    static constexpr size_t kBytes = (size_t)2 * (kM + kN) * kLdsStride * 2;
    static constexpr bool kAllStageW = 2 * kN == kT;       // every thread decodes a half row
    static_assert(W % WM == 0 && kXP % 4 == 0 && kXP > 0 && 2 * kN <= kT && (2 * kN) % 64 == 0,
                  "staging shares");
};

// WD: register stages of code loads in flight (4 or 8); K steps run in groups of WD.
// KG: groups of W waves that split the K steps (interleaved: group g takes steps
// g, g + KG, ...), each with LDS stages of its own, for more waves per SIMD on the
// same tile; their partial sums meet in LDS at the end, added in group order, so
// results do not depend on timing.  The caller makes K / 64 a multiple of KG, so
// every group passes the same barriers.
template <int W, int WM, int TM, int TN, int WD, int KG = 1>
__global__ __launch_bounds__(64 * W * KG) void k_linear_lds(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                       const uint8_t* __restrict__ packed,
                                                       const uint8_t* __restrict__ scales,
                                                       const float* __restrict__ gs_in, int64_t N,
                                                       const uint16_t* __restrict__ bias, uint16_t* __restrict__ y,
                                                       int64_t ldy)
{
    using Tile = LdsTile<W, WM, TM, TN>;
    constexpr int kM = Tile::kM, kN = Tile::kN, kT = Tile::kT, kXP = Tile::kXP;
    static_assert(KG == 1 || KG == 2, "K groups");
    static_assert(KG == 1 || (size_t)W * TM * TN * 16 * 64 * sizeof(float) <= KG * Tile::kBytes,
                  "partial sums fit the stages");
    __shared__ float sd_of[128];
    const int grp = KG == 1 ? 0 : __builtin_amdgcn_readfirstlane((int)threadIdx.x / kT);
    uint16_t* xs = reinterpret_cast<uint16_t*>(lin_lds + grp * Tile::kBytes);   // [2][kM][kLdsStride]
    uint16_t* ws = xs + 2 * kM * kLdsStride;                                      // [2][kN][kLdsStride]
    const float gs = *gs_in;
    if (threadIdx.x < 128)
        sd_of[threadIdx.x] = e4m3_decode(threadIdx.x) / gs;

    // from here on, tid and wave count within the K group
    const int tid = threadIdx.x - grp * kT, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int c = lane & 31, h = lane >> 5;
    const int wm = wave % WM, wn = wave / WM;
    const bool wstage = Tile::kAllStageW || wave < 2 * kN / 64;     // this wave decodes weight rows
    // XCD-aware order: workgroups go to the 8 XCDs round-robin by id; XCD k takes a
    // contiguous run of weight tiles, x tile by x tile, so the workgroups running on
    // one XCD at a time share their x tile's K slabs in that XCD's L2.
    uint32_t bx = blockIdx.x, by = blockIdx.y;
    if (NVFP4_LIN_LDS_REMAP && gridDim.y % 8 == 0) {
        const uint32_t w = blockIdx.x + blockIdx.y * gridDim.x;
        const uint32_t l = w / 8, per = gridDim.y / 8;               // weight tiles per XCD
        bx = l / per;
        by = (w % 8) * per + l % per;
    }
    const int64_t m0 = (int64_t)bx * kM, n0 = (int64_t)by * kN;

    // this thread's share of the staging: x rows m0 + tid / 8 + (kT / 8) j (j < kXP)
    // at columns 8 (tid % 8) of the step; weight row n0 + tid / 2, the codes of
    // columns 32 (tid % 2) .. + 32 of the step.  Rows past M read row M - 1 and
    // weight rows past N read row N - 1: they feed only output elements that are
    // not stored, and every load stays unconditional.
#if NVFP4_LIN_LDS_BUF
    // Buffer loads on resources based at the workgroup's tile: a 32-bit lane offset
    // fixed for the whole loop plus the step's offset in a scalar register, so the
    // K loop spends no VALU on addresses (the host keeps K below 2^22, so that
    // 256 rows of K bf16 stay below 2^31 bytes).
    const int64_t mrows = M - m0 < kM ? M - m0 : kM, nrows = N - n0 < kN ? N - n0 : kN;
    const __amdgpu_buffer_rsrc_t xres = tile_resource(x + m0 * K, mrows * K * 2);
    const __amdgpu_buffer_rsrc_t wres = tile_resource(packed + n0 * (K / 2), nrows * (K / 2));
    const __amdgpu_buffer_rsrc_t sres = tile_resource(scales + n0 * (K / 16), nrows * (K / 16));
    uint32_t xoff[kXP];
#pragma unroll
    for (int j = 0; j < kXP; ++j) {
        const int64_t r = tid / 8 + (kT / 8) * j;
        xoff[j] = (uint32_t)(((r < mrows ? r : mrows - 1) * K + 8 * (tid % 8) + grp * kLdsK) * 2);
    }
    const int wr = tid >> 1, wh = tid & 1;
    const int64_t wrl = wr < nrows ? wr : nrows - 1;
    const uint32_t woff = (uint32_t)(wrl * (K / 2) + 16 * wh + grp * (kLdsK / 2));
    const uint32_t soff = (uint32_t)(wrl * (K / 16) + 2 * wh + grp * (kLdsK / 16));

    // st counts the group's own steps (K step KG st + grp)
    auto load_x = [&](int64_t st, uint4 (&v)[kXP]) __attribute__((always_inline)) {
        const int so = (int)(st * (KG * kLdsK * 2));
#pragma unroll
        for (int j = 0; j < kXP; ++j)
            v[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xres, xoff[j], so, 0));
    };
    auto load_w = [&](int64_t st, uint4& cw, uint32_t& sc) __attribute__((always_inline)) {
        if (!wstage)
            return;
        cw = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wres, woff, (int)(st * (KG * kLdsK / 2)), 0));
        sc = __builtin_amdgcn_raw_buffer_load_b16(sres, soff, (int)(st * (KG * kLdsK / 16)), 0);
    };
#else
    const uint16_t* xrow[kXP];
#pragma unroll
    for (int j = 0; j < kXP; ++j) {
        const int64_t m = m0 + tid / 8 + (kT / 8) * j;
        xrow[j] = x + (m < M ? m : M - 1) * K + 8 * (tid % 8) + grp * kLdsK;
    }
    const int wr = tid >> 1, wh = tid & 1;
    const int64_t wrn = n0 + wr < N ? n0 + wr : N - 1;
    const uint8_t* wrow = packed + wrn * (K / 2) + 16 * wh + grp * (kLdsK / 2);
    const uint8_t* srow = scales + wrn * (K / 16) + 2 * wh + grp * (kLdsK / 16);

    // st counts the group's own steps (K step KG st + grp)
    auto load_x = [&](int64_t st, uint4 (&v)[kXP]) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < kXP; ++j)
            v[j] = *reinterpret_cast<const uint4*>(xrow[j] + st * (KG * kLdsK));
    };
    auto load_w = [&](int64_t st, uint4& cw, uint32_t& sc) __attribute__((always_inline)) {
        if (!wstage)
            return;
        cw = *reinterpret_cast<const uint4*>(wrow + st * (KG * kLdsK / 2));
        sc = *reinterpret_cast<const uint16_t*>(srow + st * (KG * kLdsK / 16));
    };
#endif
    // piece q (0..3) of the staging of one step into buffer buf: a quarter of the
    // thread's x pieces and one decoded dword of its codes (eight weights)
    auto stage = [&](int buf, int q, const uint4 (&xv)[kXP], const uint4& cw, uint32_t sc)
        __attribute__((always_inline)) {
#pragma unroll
        for (int jj = 0; jj < kXP / 4; ++jj) {
            const int j = (kXP / 4) * q + jj;
            *reinterpret_cast<uint4*>(xs + (buf * kM + tid / 8 + (kT / 8) * j) * kLdsStride + 8 * (tid % 8)) =
                xv[j];
        }
        if (wstage) {
            const float sd = sd_of[(sc >> (8 * (q / 2))) & 0x7Fu];
            *reinterpret_cast<uint4*>(ws + (buf * kN + wr) * kLdsStride + 32 * wh + 8 * q) =
                decode_half(dword_of(cw, q), sd);
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int t = 0; t < TN; ++t)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                acc[i][t][j] = 0.0f;
    // slice q (16 of the step's 64 K) of this stage's MFMAs from buffer buf
    // the MFMA operands of slice q (16 of the step's 64 K) from buffer buf
    auto read_slice = [&](int buf, int q, bf16x8 (&a)[TM], bf16x8 (&b)[TN]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
            a[i] = *reinterpret_cast<const bf16x8*>(xs + (buf * kM + 32 * (TM * wm + i) + c) * kLdsStride +
                                                    16 * q + 8 * h);
#pragma unroll
        for (int t = 0; t < TN; ++t)
            b[t] = *reinterpret_cast<const bf16x8*>(ws + (buf * kN + 32 * (TN * wn + t) + c) * kLdsStride +
                                                    16 * q + 8 * h);
    };
    auto mma = [&](const bf16x8 (&a)[TM], const bf16x8 (&b)[TN]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int t = 0; t < TN; ++t)
                acc[i][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[t], acc[i][t], 0, 0, 0);
    };
    auto mma_slice = [&](int buf, int q) __attribute__((always_inline)) {
        bf16x8 a[TM], b[TN];
        read_slice(buf, q, a, b);
        mma(a, b);
    };
    // Pipelined operands (the 4-wave tile, which has the registers for it): slice
    // q + 1's operands are read into the other of two register sets before slice
    // q's MFMAs issue, so those MFMAs wait on no LDS read.
    constexpr bool Pipe = NVFP4_LIN_LDS_PIPE != 0 && W == 4;
    bf16x8 fa[2][TM], fb[2][TN];

    const int64_t steps = K / kLdsK / KG;
    constexpr int kLdsWDepth = WD;
    uint4 xr[kLdsXDepth][kXP];
    uint4 cr[kLdsWDepth];
    uint32_t sr[kLdsWDepth];
#pragma unroll
    for (int d = 0; d < kLdsWDepth; ++d)
        if (d < steps)
            load_w(d, cr[d], sr[d]);
#pragma unroll
    for (int d = 0; d < kLdsXDepth; ++d)
        if (d < steps)
            load_x(d, xr[d]);
    __syncthreads();                                          // sd_of
#pragma unroll
    for (int q = 0; q < 4; ++q)
        stage(0, q, xr[0], cr[0], sr[0]);
    if (kLdsXDepth < steps)
        load_x(kLdsXDepth, xr[0]);
    if (kLdsWDepth < steps)
        load_w(kLdsWDepth, cr[0], sr[0]);
    __syncthreads();
    static_assert((WD == 4 || WD == 8) && kLdsXDepth == 2, "ring indices repeat every WD steps");
    // step st0 + D of a group of WD: the ring slots are compile-time constants.
    // Checked (the last, partial group): steps past the end are skipped, and
    // neither staging nor loads run for steps that do not exist.  Unchecked (a
    // group of WD whole steps): the step is one basic block, so the compiler
    // can issue a slice's LDS reads under the previous slice's MFMAs; staging
    // always runs (after the last step it fills a buffer that nothing reads,
    // whose last reads ended at the previous barrier) and loads clamp their step.
    auto step = [&](int64_t st0, auto dc, auto checked) __attribute__((always_inline)) {
        constexpr int D = decltype(dc)::value;
        constexpr bool C = decltype(checked)::value;
        constexpr int cur = D & 1, nxt = cur ^ 1, xn = (D + 1) % kLdsXDepth, wnx = (D + 1) % kLdsWDepth;
        const int64_t st = st0 + D;
        if (C && st >= steps)
            return;
        const bool more = !C || st + 1 < steps;
        // slice q of this stage's MFMAs, then piece q of the next stage's staging
        auto slice = [&](auto qc) __attribute__((always_inline)) {
            constexpr int q = decltype(qc)::value;
            if (Pipe) {
                if (q == 0)
                    read_slice(cur, 0, fa[0], fb[0]);
                if (q < 3)
                    read_slice(cur, q + 1, fa[(q + 1) & 1], fb[(q + 1) & 1]);
                mma(fa[q & 1], fb[q & 1]);
            } else {
                mma_slice(cur, q);
            }
            if (more)
                stage(nxt, q, xr[xn], cr[wnx], sr[wnx]);
        };
        slice(std::integral_constant<int, 0>{});
        slice(std::integral_constant<int, 1>{});
        slice(std::integral_constant<int, 2>{});
        slice(std::integral_constant<int, 3>{});
        if (!C) {
            const int64_t sx = st + 1 + kLdsXDepth, sw = st + 1 + kLdsWDepth;
            load_x(sx < steps ? sx : steps - 1, xr[xn]);
            load_w(sw < steps ? sw : steps - 1, cr[wnx], sr[wnx]);
        } else {
            if (st + 1 + kLdsXDepth < steps)
                load_x(st + 1 + kLdsXDepth, xr[xn]);
            if (st + 1 + kLdsWDepth < steps)
                load_w(st + 1 + kLdsWDepth, cr[wnx], sr[wnx]);
        }
        __syncthreads();
    };
    constexpr bool kFlat = NVFP4_LIN_LDS_FLAT != 0;
    int64_t st0 = 0;
    if (kFlat) {
        for (; st0 + kLdsWDepth <= steps; st0 += kLdsWDepth)
            for_each_index([&](auto dc) __attribute__((always_inline)) { step(st0, dc, std::false_type{}); },
                           std::make_index_sequence<WD>{});
    }
    for (; st0 < steps; st0 += kLdsWDepth)
        for_each_index([&](auto dc) __attribute__((always_inline)) { step(st0, dc, std::true_type{}); },
                       std::make_index_sequence<WD>{});

    if (KG == 2) {
        // group 1's partial sums through LDS (the K loop's last barrier ended every
        // read of the stages), added to group 0's
        float* part = reinterpret_cast<float*>(lin_lds);          // [W][TM][TN][16][64]
        if (grp == 1) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int t = 0; t < TN; ++t)
#pragma unroll
                    for (int j = 0; j < 16; ++j)
                        part[(((wave * TM + i) * TN + t) * 16 + j) * 64 + lane] = acc[i][t][j];
        }
        __syncthreads();
        if (grp == 1)
            return;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int t = 0; t < TN; ++t)
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    acc[i][t][j] += part[(((wave * TM + i) * TN + t) * 16 + j) * 64 + lane];
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int t = 0; t < TN; ++t) {
            const int64_t n = n0 + 32 * (TN * wn + t) + c;
            if (n >= N)
                continue;
            const float b = bias ? bf16_value(bias[n]) : 0.0f;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int64_t m = m0 + 32 * (TM * wm + i) + (j % 4) + 8 * (j / 4) + 4 * h;
                if (m < M) {
                    const f32x2 o = {acc[i][t][j] + b, 0.0f};
                    y[m * ldy + n] = (uint16_t)(__builtin_bit_cast(uint32_t, __builtin_convertvector(o, bf16x2)) & 0xFFFFu);
                }
            }
        }
    }
}

}  // namespace

#endif  // NVFP4_LINEAR_HPP
