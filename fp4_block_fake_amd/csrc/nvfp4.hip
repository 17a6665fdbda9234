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
// * Every kernel streams HBM: 2-6 bytes per element, a few dozen integer ops.
//   There is no contraction, so no MFMA; the limits are HBM bandwidth and the
//   VALU issue rate (about 20 lane-ops per element at 8 TB/s for fake-quant).
// * One lane owns one 16-element block (two 16-byte loads).  The block max is
//   taken from the lane's own registers with packed 16-bit max on the
//   magnitude fields; no cross-lane traffic is needed per block.
// * The per-element IEEE divide x / sq is replaced by integer compares that
//   give bit-identical codes (see "Decision thresholds" below).  Everything
//   that depends only on the E4M3 scale byte S (the thresholds and the eight
//   bf16 outputs of the block) is built once per workgroup for all 128 bytes
//   into a 6 KB LDS table, so a block costs one scale computation and one LDS
//   lookup.
// * Workgroups are persistent (a few per CU) and walk the tensor with a grid
//   stride, which amortises the table build over many blocks.
// * The per-tensor amax is a separate streaming pass with one atomic max per
//   workgroup; the quantizing kernels read it from device memory, so a fused
//   call never returns to the host.
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

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "nvfp4.h"

namespace {

// Launch shape and cache hints per kernel.  The defaults come from sweeps on
// MI355X (c5 weight, 470 MB); the macros let a build be re-tuned without
// editing the kernels.
#ifndef NVFP4_UNROLL
#define NVFP4_UNROLL 2            // blocks per lane per iteration: fake-quant, pack
#endif
#ifndef NVFP4_DQ_UNROLL
#define NVFP4_DQ_UNROLL 4         // blocks per lane per iteration: unpack
#endif
#ifndef NVFP4_AMAX_UNROLL
#define NVFP4_AMAX_UNROLL 8       // 16-byte vectors per lane per amax chunk
#endif
#ifndef NVFP4_AMAX_WG_PER_CU
#define NVFP4_AMAX_WG_PER_CU 4    // persistent workgroups per CU
#endif
#ifndef NVFP4_FQ_WG_PER_CU
#define NVFP4_FQ_WG_PER_CU 32
#endif
#ifndef NVFP4_QP_WG_PER_CU
#define NVFP4_QP_WG_PER_CU 32
#endif
#ifndef NVFP4_DQ_WG_PER_CU
#define NVFP4_DQ_WG_PER_CU 64
#endif
// 1: the quantizing passes walk the tensor from its end, so they start on the
// data the amax pass read last.  This pays only when the amax pass leaves x in
// the Infinity Cache, i.e. with NVFP4_AMAX_NT 0; streaming amax loads win more.
#ifndef NVFP4_REVERSE
#define NVFP4_REVERSE 0
#endif
// non-temporal (streaming) hints on loads (LD) and stores (ST)
#ifndef NVFP4_AMAX_NT
#define NVFP4_AMAX_NT 1
#endif
#ifndef NVFP4_FQ_NT_LD
#define NVFP4_FQ_NT_LD 0
#endif
#ifndef NVFP4_FQ_NT_ST
#define NVFP4_FQ_NT_ST 0
#endif
#ifndef NVFP4_QP_NT_LD
#define NVFP4_QP_NT_LD 1
#endif
#ifndef NVFP4_QP_NT_ST
#define NVFP4_QP_NT_ST 1
#endif
#ifndef NVFP4_DQ_NT_ST
#define NVFP4_DQ_NT_ST 0
#endif

constexpr int kThreads = 256;                    // 4 waves of 64
constexpr int kUnroll = NVFP4_UNROLL;
constexpr int kDqUnroll = NVFP4_DQ_UNROLL;
constexpr int kAmaxUnroll = NVFP4_AMAX_UNROLL;
constexpr bool kReverse = NVFP4_REVERSE != 0;

constexpr float kEps = 1e-12f;    // clamp of the amax and of the block scale
constexpr float kGsNumerator = 2688.0f;  // E4M3 max 448 times E2M1 max 6

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- packed 16-bit helpers

__device__ __forceinline__ u16x2 h2(uint32_t v) { return __builtin_bit_cast(u16x2, v); }
__device__ __forceinline__ uint32_t w32(u16x2 v) { return __builtin_bit_cast(uint32_t, v); }

__device__ __forceinline__ uint32_t pk_max(uint32_t a, uint32_t b)
{
    return w32(__builtin_elementwise_max(h2(a), h2(b)));
}
__device__ __forceinline__ uint32_t pk_sub(uint32_t a, uint32_t b) { return w32(h2(a) - h2(b)); }
// bit 15 of each half moved to bit 0: for a, b < 0x8000, pk_top(pk_sub(a, b)) = [a < b]
__device__ __forceinline__ uint32_t pk_top(uint32_t a) { return w32(h2(a) >> (u16x2)15); }
__device__ __forceinline__ uint32_t pk_mad(uint32_t a, uint32_t b, uint32_t c)
{
    return w32(h2(a) * h2(b) + h2(c));
}

// ---------------------------------------------------------------- memory helpers

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <bool NT>
__device__ __forceinline__ uint4 load16(const uint4* p)
{
    if (NT)
        return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
    return *p;
}
template <bool NT>
__device__ __forceinline__ void store16(uint4* p, uint4 v)
{
    if (NT)
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4*>(p));
    else
        *p = v;
}
template <bool NT>
__device__ __forceinline__ void store8(uint2* p, uint2 v)
{
    if (NT)
        __builtin_nontemporal_store(__builtin_bit_cast(u32x2, v), reinterpret_cast<u32x2*>(p));
    else
        *p = v;
}

// ---------------------------------------------------------------- scalar number formats

__device__ __forceinline__ float global_scale_of(float amax)
{
    float a = amax < kEps ? kEps : amax;
    return kGsNumerator / a;          // IEEE binary32 divide (no fast-math in this build)
}

// Non-negative binary32 -> E4M3 byte, round-to-nearest-even, saturating at 0x7E (448).
__device__ __forceinline__ uint32_t e4m3_encode(float v)
{
    uint32_t u = __float_as_uint(v);
    // normal E4M3 (v >= 2^-6): round the binary32 significand to 3 bits, rebias 127 -> 7
    uint32_t normal = ((u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20) - (120u << 3);
    // subnormal E4M3: multiples of 2^-9; v * 512 is exact, rint rounds half to even
    uint32_t sub = (uint32_t)__builtin_rintf(v * 512.0f);
    uint32_t s = v < 0x1p-6f ? sub : normal;
    return s < 0x7Eu ? s : 0x7Eu;
}

// E4M3 byte 0..0x7F (sign clear) -> value.  0x7F (NaN) never reaches here as a scale.
__device__ __forceinline__ float e4m3_decode(uint32_t s)
{
    return s >= 8u ? __uint_as_float((s << 20) + (120u << 23)) : (float)s * 0x1p-9f;
}

// binary32 -> bf16 bits, round-to-nearest-even.
__device__ __forceinline__ uint32_t bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)
        return (u >> 16) | 0x40u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Bits of the largest bf16 value <= t (t > 0, an exact binary64), and whether t is one.
__device__ __forceinline__ uint32_t bf16_floor_bits(double t, bool& exact)
{
    const double kMax = 0x1.fep127;   // largest finite bf16
    if (t >= kMax) {
        exact = (t == kMax);
        return 0x7F7Fu;
    }
    if (t < 0x1p-126) {               // bf16 subnormals are multiples of 2^-133
        double k = __builtin_floor(t * 0x1p133);
        exact = (k == t * 0x1p133);
        return (uint32_t)k;
    }
    uint64_t b = (uint64_t)__double_as_longlong(t);
    exact = (b & ((1ull << 45) - 1)) == 0;
    return (uint32_t)(b >> 45) - (896u << 7);  // binary64 exponent bias 1023 -> 127
}

// first bf16 bit pattern strictly above t / at or above t, capped at +inf (0x7F80)
__device__ __forceinline__ uint32_t first_above(double t)
{
    bool exact;
    uint32_t f = bf16_floor_bits(t, exact) + 1u;
    return f < 0x7F80u ? f : 0x7F80u;
}
__device__ __forceinline__ uint32_t first_at_or_above(double t)
{
    bool exact;
    uint32_t f = bf16_floor_bits(t, exact) + (exact ? 0u : 1u);
    return f < 0x7F80u ? f : 0x7F80u;
}

// ---------------------------------------------------------------- per-scale-byte table
//
// Entry for scale byte S (12 dwords, three 16-byte LDS reads):
//   [0] t4 | t4<<16            [1] t6 | t6<<16           [2] (t2-t6) | (t2-t6)<<16
//   [3] (t0-1) | (t0-1)<<16    [4] t7 | t5<<16           [5] t3 | t1<<16
//   [6..9] low and high bytes of the eight bf16 outputs, ordered by k = 7 - idx
//   [10..11] unused
// t_i (i = 1..7) is the smallest magnitude bit pattern whose E2M1 index is >= i;
// t0 the smallest whose quotient is nonzero.
constexpr int kEntryVec = 3;   // uint4 per entry

__device__ void build_entry(uint32_t s, float gs, uint4* dst)
{
    const float sd = e4m3_decode(s) / gs;          // decoded block scale
    const float sq = sd < kEps ? kEps : sd;        // the divisor of the elements
    const double q = (double)sq;
    const uint32_t t0 = first_above(q * 0x1p-150);
    const uint32_t t1 = first_above((0.25 + 0x1p-26) * q);
    const uint32_t t2 = first_at_or_above((0.75 - 0x1p-25) * q);
    const uint32_t t3 = first_above((1.25 + 0x1p-24) * q);
    const uint32_t t4 = first_at_or_above((1.75 - 0x1p-24) * q);
    const uint32_t t5 = first_above((2.5 + 0x1p-23) * q);
    const uint32_t t6 = first_at_or_above((3.5 - 0x1p-23) * q);
    const uint32_t t7 = first_above((5.0 + 0x1p-22) * q);
    // outputs by k = 7 - idx: magnitudes 6, 4, 3, 2, 1.5, 1, 0.5, 0 times sd
    const uint32_t o0 = bf16_bits(6.0f * sd), o1 = bf16_bits(4.0f * sd);
    const uint32_t o2 = bf16_bits(3.0f * sd), o3 = bf16_bits(2.0f * sd);
    const uint32_t o4 = bf16_bits(1.5f * sd), o5 = bf16_bits(1.0f * sd);
    const uint32_t o6 = bf16_bits(0.5f * sd), o7 = bf16_bits(0.0f * sd);
    const uint32_t d26 = (t2 - t6) & 0xFFFFu;
    dst[0] = make_uint4(t4 * 0x10001u, t6 * 0x10001u, d26 * 0x10001u, (t0 - 1u) * 0x10001u);
    dst[1] = make_uint4(t7 | (t5 << 16), t3 | (t1 << 16),
                        (o0 & 0xFFu) | (o1 & 0xFFu) << 8 | (o2 & 0xFFu) << 16 | (o3 & 0xFFu) << 24,
                        (o4 & 0xFFu) | (o5 & 0xFFu) << 8 | (o6 & 0xFFu) << 16 | (o7 & 0xFFu) << 24);
    dst[2] = make_uint4((o0 >> 8) | (o1 >> 8) << 8 | (o2 >> 8) << 16 | (o3 >> 8) << 24,
                        (o4 >> 8) | (o5 >> 8) << 8 | (o6 >> 8) << 16 | (o7 >> 8) << 24, 0u, 0u);
}

struct Entry {
    uint32_t t4, t6, d26, t0m1, tab_lo, tab_hi, lo_a, lo_b, hi_a, hi_b;
};

__device__ __forceinline__ Entry load_entry(const uint4* table, uint32_t s, bool with_outputs)
{
    const uint4* e = table + s * kEntryVec;
    uint4 a = e[0], b = e[1];
    Entry r{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w, 0u, 0u};
    if (with_outputs) {
        uint4 c = e[2];
        r.hi_a = c.x;
        r.hi_b = c.y;
    }
    return r;
}

// k = 7 - idx for the two magnitudes m (15-bit fields) of one dword
__device__ __forceinline__ uint32_t reversed_index(uint32_t m, const Entry& e)
{
    uint32_t n4 = pk_top(pk_sub(m, e.t4));                   // [m < t4]
    uint32_t ta = pk_mad(n4, e.d26, e.t6);                   // n4 ? t2 : t6
    uint32_t na = pk_top(pk_sub(m, ta));
    uint32_t j = pk_mad(n4, 0x00020002u, na);                // 0..3
    uint32_t sel = pk_mad(j, 0x02020202u, 0x01000100u);      // bytes 2j, 2j+1 per half
    uint32_t tb = __builtin_amdgcn_perm(e.tab_hi, e.tab_lo, sel);  // t7, t5, t3, t1 by j
    uint32_t nb = pk_top(pk_sub(m, tb));
    return pk_mad(j, 0x00020002u, nb);
}

// Sign bits (15 and 31) of the two codes: x negative and |x| >= t0.
__device__ __forceinline__ uint32_t code_signs(uint32_t w, uint32_t m, const Entry& e)
{
    return w & pk_sub(e.t0m1, m) & 0x80008000u;
}

// Two bf16 inputs -> two fake-quantized bf16 outputs.
__device__ __forceinline__ uint32_t fake_quant_pair(uint32_t w, const Entry& e)
{
    const uint32_t m = w & 0x7FFF7FFFu;
    const uint32_t k = reversed_index(m, e);
    const uint32_t sel = k | (k << 8);
    const uint32_t lo = __builtin_amdgcn_perm(e.lo_b, e.lo_a, sel);
    const uint32_t hi = __builtin_amdgcn_perm(e.hi_b, e.hi_a, sel);
    return (hi & 0xFF00FF00u) | (lo & 0x00FF00FFu) | code_signs(w, m, e);
}

// Two bf16 inputs -> one byte: code of the first in the low nibble, second in the high.
__device__ __forceinline__ uint32_t code_byte(uint32_t w, const Entry& e)
{
    const uint32_t m = w & 0x7FFF7FFFu;
    const uint32_t c = (reversed_index(m, e) ^ 0x00070007u) | (code_signs(w, m, e) >> 12);
    return (c | (c >> 12)) & 0xFFu;
}

// Block scale byte of a block from its eight dwords.
__device__ __forceinline__ uint32_t block_scale_byte(const uint32_t (&w)[8], float gs)
{
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        mx = pk_max(mx, w[i] & 0x7FFF7FFFu);
    const uint32_t bm = max(mx & 0xFFFFu, mx >> 16);
    const float bamax = __uint_as_float(bm << 16);
    return e4m3_encode((bamax / 6.0f) * gs);
}

__device__ __forceinline__ void unpack8(const uint4& a, const uint4& b, uint32_t (&w)[8])
{
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
}

// ---------------------------------------------------------------- kernels

// i-th block of a pass (or -1 past the end); the pass runs backwards when kReverse.
__device__ __forceinline__ int64_t walk(int64_t i, int64_t nblocks)
{
    if (i >= nblocks)
        return -1;
    return kReverse ? nblocks - 1 - i : i;
}

__global__ void k_set_scalar(float* p, float v) { *p = v; }

struct AmaxGroup {
    const uint4* vec[NVFP4_AMAX_GROUP_MAX];        // 16-byte-aligned starts
    int64_t nvec[NVFP4_AMAX_GROUP_MAX];            // numel / 8
    int64_t chunk_end[NVFP4_AMAX_GROUP_MAX];       // running sum of chunks
    const uint16_t* tail[NVFP4_AMAX_GROUP_MAX];    // last numel % 8 values
    int32_t ntail[NVFP4_AMAX_GROUP_MAX];
    int32_t count;
};

// max |x| over a group of tensors; one signed-integer atomic max per workgroup on
// the fp32 bits of the result (non-negative floats order like their bits, and a
// negative prior value loses to any of them).
__global__ __launch_bounds__(kThreads) void k_amax(AmaxGroup g, float* out)
{
    constexpr int64_t kChunk = (int64_t)kThreads * kAmaxUnroll;
    uint32_t mx = 0;
    const int64_t total = g.chunk_end[g.count - 1];
    // chunks only grow along the loop, so the current tensor is cached and
    // advanced instead of searched for on every chunk
    int t = 0;
    int64_t begin = 0, end = g.chunk_end[0], n = g.nvec[0];
    const uint4* __restrict__ src = g.vec[0];
    for (int64_t c = blockIdx.x; c < total; c += gridDim.x) {
        while (c >= end) {
            ++t;
            begin = end;
            end = g.chunk_end[t];
            n = g.nvec[t];
            src = g.vec[t];
        }
        const int64_t first = (c - begin) * kChunk + threadIdx.x;
        uint4 v[kAmaxUnroll];
#pragma unroll
        for (int u = 0; u < kAmaxUnroll; ++u) {
            const int64_t i = first + (int64_t)u * kThreads;
            v[u] = i < n ? load16<NVFP4_AMAX_NT != 0>(src + i) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < kAmaxUnroll; ++u) {
            mx = pk_max(mx, v[u].x & 0x7FFF7FFFu);
            mx = pk_max(mx, v[u].y & 0x7FFF7FFFu);
            mx = pk_max(mx, v[u].z & 0x7FFF7FFFu);
            mx = pk_max(mx, v[u].w & 0x7FFF7FFFu);
        }
    }
    if (blockIdx.x == 0) {
        for (int t = 0; t < g.count; ++t)
            if ((int)threadIdx.x < g.ntail[t])
                mx = pk_max(mx, g.tail[t][threadIdx.x] & 0x7FFFu);
    }
    uint32_t m = max(mx & 0xFFFFu, mx >> 16);
    // wave reduction over 64 lanes
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
    __shared__ uint32_t wave_max[kThreads / 64];
    if ((threadIdx.x & 63) == 0)
        wave_max[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = wave_max[0];
#pragma unroll
        for (int i = 1; i < kThreads / 64; ++i)
            r = max(r, wave_max[i]);
        atomicMax(reinterpret_cast<int*>(out), (int)(r << 16));
    }
}

__global__ __launch_bounds__(kThreads) void k_fake_quant(const uint4* __restrict__ x, uint4* y,
                                                         int64_t nblocks,
                                                         const float* __restrict__ amax)
{
    __shared__ uint4 table[128 * kEntryVec];
    const float gs = global_scale_of(*amax);
    if (threadIdx.x < 128)
        build_entry(threadIdx.x, gs, table + threadIdx.x * kEntryVec);
    __syncthreads();

    const int64_t stride = (int64_t)gridDim.x * kThreads * kUnroll;
    for (int64_t base = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; base < nblocks;
         base += stride) {
        uint4 v[kUnroll][2];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t b = walk(base + (int64_t)u * kThreads, nblocks);
            if (b >= 0) {
                v[u][0] = load16<NVFP4_FQ_NT_LD != 0>(x + 2 * b);
                v[u][1] = load16<NVFP4_FQ_NT_LD != 0>(x + 2 * b + 1);
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t b = walk(base + (int64_t)u * kThreads, nblocks);
            if (b >= 0) {
                uint32_t w[8];
                unpack8(v[u][0], v[u][1], w);
                const Entry e = load_entry(table, block_scale_byte(w, gs), true);
                uint32_t o[8];
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    o[i] = fake_quant_pair(w[i], e);
                store16<NVFP4_FQ_NT_ST != 0>(y + 2 * b, make_uint4(o[0], o[1], o[2], o[3]));
                store16<NVFP4_FQ_NT_ST != 0>(y + 2 * b + 1, make_uint4(o[4], o[5], o[6], o[7]));
            }
        }
    }
}

__global__ __launch_bounds__(kThreads) void k_quantize_pack(const uint4* __restrict__ x,
                                                            uint2* __restrict__ packed,
                                                            uint8_t* __restrict__ scales,
                                                            float* __restrict__ gs_out,
                                                            int64_t nblocks,
                                                            const float* __restrict__ amax)
{
    __shared__ uint4 table[128 * kEntryVec];
    const float gs = global_scale_of(*amax);
    if (threadIdx.x < 128)
        build_entry(threadIdx.x, gs, table + threadIdx.x * kEntryVec);
    if (blockIdx.x == 0 && threadIdx.x == 0)
        *gs_out = gs;
    __syncthreads();

    const int64_t stride = (int64_t)gridDim.x * kThreads * kUnroll;
    for (int64_t base = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; base < nblocks;
         base += stride) {
        uint4 v[kUnroll][2];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t b = walk(base + (int64_t)u * kThreads, nblocks);
            if (b >= 0) {
                v[u][0] = load16<NVFP4_QP_NT_LD != 0>(x + 2 * b);
                v[u][1] = load16<NVFP4_QP_NT_LD != 0>(x + 2 * b + 1);
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t b = walk(base + (int64_t)u * kThreads, nblocks);
            if (b >= 0) {
                uint32_t w[8];
                unpack8(v[u][0], v[u][1], w);
                const uint32_t s = block_scale_byte(w, gs);
                const Entry e = load_entry(table, s, false);
                uint32_t c[8];
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    c[i] = code_byte(w[i], e);
                store8<NVFP4_QP_NT_ST != 0>(packed + b, make_uint2(c[0] | c[1] << 8 | c[2] << 16 | c[3] << 24,
                                                        c[4] | c[5] << 8 | c[6] << 16 | c[7] << 24));
                scales[b] = (uint8_t)s;
            }
        }
    }
}

// Unpack table: per scale byte, the low and high bytes of bf16(M_i * sd), i = 0..7.
__device__ void build_unpack_entry(uint32_t s, float gs, uint4* dst)
{
    const float sd = e4m3_decode(s) / gs;
    uint32_t o[8];
    const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
#pragma unroll
    for (int i = 0; i < 8; ++i)
        o[i] = bf16_bits(mag[i] * sd);
    *dst = make_uint4((o[0] & 0xFFu) | (o[1] & 0xFFu) << 8 | (o[2] & 0xFFu) << 16 | (o[3] & 0xFFu) << 24,
                      (o[4] & 0xFFu) | (o[5] & 0xFFu) << 8 | (o[6] & 0xFFu) << 16 | (o[7] & 0xFFu) << 24,
                      (o[0] >> 8) | (o[1] >> 8) << 8 | (o[2] >> 8) << 16 | (o[3] >> 8) << 24,
                      (o[4] >> 8) | (o[5] >> 8) << 8 | (o[6] >> 8) << 16 | (o[7] >> 8) << 24);
}

// Eight codes (one dword of packed nibbles) -> eight bf16 values in four dwords.
__device__ __forceinline__ void unpack_dword(uint32_t p, const uint4& t, uint32_t* out)
{
    const uint32_t lo = p & 0x07070707u;           // magnitude index of even columns
    const uint32_t hi = (p >> 4) & 0x07070707u;    // ... of odd columns
    const uint32_t sl = (p << 4) & 0x80808080u;    // sign of even columns at bit 7
    const uint32_t sh = p & 0x80808080u;           // sign of odd columns at bit 7
#pragma unroll
    for (uint32_t q = 0; q < 4; ++q) {
        const uint32_t sel = __builtin_amdgcn_perm(hi, lo, q | q << 8 | (4u + q) << 16 | (4u + q) << 24);
        const uint32_t vl = __builtin_amdgcn_perm(t.y, t.x, sel);
        const uint32_t vh = __builtin_amdgcn_perm(t.w, t.z, sel);
        const uint32_t sg = __builtin_amdgcn_perm(sh, sl, 0x0Cu | q << 8 | 0x0Cu << 16 | (4u + q) << 24);
        out[q] = (vh & 0xFF00FF00u) | (vl & 0x00FF00FFu) | sg;
    }
}

__global__ __launch_bounds__(kThreads) void k_dequant_unpack(const uint2* __restrict__ packed,
                                                             const uint8_t* __restrict__ scales,
                                                             const float* __restrict__ gs_in,
                                                             uint4* __restrict__ y, int64_t nblocks)
{
    __shared__ uint4 table[128];
    const float gs = *gs_in;
    if (threadIdx.x < 128)
        build_unpack_entry(threadIdx.x, gs, table + threadIdx.x);
    __syncthreads();

    const int64_t stride = (int64_t)gridDim.x * kThreads * kDqUnroll;
    for (int64_t base = (int64_t)blockIdx.x * kThreads * kDqUnroll + threadIdx.x; base < nblocks;
         base += stride) {
        uint2 p[kDqUnroll];
        uint32_t s[kDqUnroll];
#pragma unroll
        for (int u = 0; u < kDqUnroll; ++u) {
            const int64_t b = base + (int64_t)u * kThreads;
            if (b < nblocks) {
                p[u] = packed[b];
                s[u] = scales[b];
            }
        }
#pragma unroll
        for (int u = 0; u < kDqUnroll; ++u) {
            const int64_t b = base + (int64_t)u * kThreads;
            if (b < nblocks) {
                const uint4 t = table[s[u] & 0x7Fu];
                uint32_t o[8];
                unpack_dword(p[u].x, t, o);
                unpack_dword(p[u].y, t, o + 4);
                store16<NVFP4_DQ_NT_ST != 0>(y + 2 * b, make_uint4(o[0], o[1], o[2], o[3]));
                store16<NVFP4_DQ_NT_ST != 0>(y + 2 * b + 1, make_uint4(o[4], o[5], o[6], o[7]));
            }
        }
    }
}

__global__ void k_observer(float* state, const float* cur, int mode, float decay)
{
    const float s = *state, c = *cur;
    float r;
    if (s < 0.0f) {
        r = c;                                     // first observation
    } else if (mode == NVFP4_OBS_STATIC_MINMAX) {
        r = c > s ? c : s;
    } else {
        const float keep = 1.0f - decay;
        const float a = keep * s;
        const float b = decay * c;
        r = a + b;                                 // no contraction: -ffp-contract=off
    }
    *state = r;
}

// ---------------------------------------------------------------- host helpers

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool overlap(const void* a, uint64_t na, const void* b, uint64_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return na && nb && x < y + nb && y < x + na;
}

nvfp4_status check_matrix(int64_t rows, int64_t cols, int64_t* numel)
{
    if (rows < 0 || cols < 16 || cols % 16 != 0)
        return NVFP4_ERR_SHAPE;
    if (rows > 0 && cols > (INT64_MAX / 4) / rows)
        return NVFP4_ERR_SHAPE;
    *numel = rows * cols;
    return NVFP4_OK;
}

unsigned persistent_grid(int64_t items, int64_t items_per_wg, int wg_per_cu)
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    const int64_t need = (items + items_per_wg - 1) / items_per_wg;
    const int64_t cap = (int64_t)cus * wg_per_cu;
    return (unsigned)(need < 1 ? 1 : (need < cap ? need : cap));
}

nvfp4_status launched()
{
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

// Enqueue max|x| of up to NVFP4_AMAX_GROUP_MAX tensors into *amax (atomic max).
nvfp4_status enqueue_amax(const void* const* xs, const int64_t* numels, int n, float* amax,
                          hipStream_t stream)
{
    AmaxGroup g{};
    constexpr int64_t kChunk = (int64_t)kThreads * kAmaxUnroll;
    int64_t chunks = 0;
    g.count = n;
    for (int i = 0; i < n; ++i) {
        g.vec[i] = static_cast<const uint4*>(xs[i]);
        g.nvec[i] = numels[i] / 8;
        g.tail[i] = static_cast<const uint16_t*>(xs[i]) + (numels[i] & ~(int64_t)7);
        g.ntail[i] = (int32_t)(numels[i] & 7);
        chunks += (g.nvec[i] + kChunk - 1) / kChunk;
        g.chunk_end[i] = chunks;
    }
    k_amax<<<persistent_grid(chunks, 1, NVFP4_AMAX_WG_PER_CU), kThreads, 0, stream>>>(g, amax);
    return launched();
}

nvfp4_status enqueue_amax_one(const void* x, int64_t numel, float* amax, hipStream_t stream)
{
    k_set_scalar<<<1, 1, 0, stream>>>(amax, 0.0f);
    nvfp4_status st = launched();
    if (st != NVFP4_OK || numel == 0)
        return st;
    return enqueue_amax(&x, &numel, 1, amax, stream);
}

}  // namespace

// ---------------------------------------------------------------- C ABI

extern "C" {

const char* nvfp4_strerror(int status)
{
    switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "a required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "bad shape (need rows >= 0, cols >= 16, cols % 16 == 0)";
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
    if (!accumulate) {
        k_set_scalar<<<1, 1, 0, s>>>(amax, 0.0f);
        if (launched() != NVFP4_OK)
            return NVFP4_ERR_HIP;
    }
    for (int first = 0; first < n; first += NVFP4_AMAX_GROUP_MAX) {
        const void* gx[NVFP4_AMAX_GROUP_MAX];
        int64_t gn[NVFP4_AMAX_GROUP_MAX];
        int k = 0;
        for (int i = first; i < n && i < first + NVFP4_AMAX_GROUP_MAX; ++i)
            if (numels[i] > 0) {
                gx[k] = xs[i];
                gn[k] = numels[i];
                ++k;
            }
        if (k == 0)
            continue;
        nvfp4_status st = enqueue_amax(gx, gn, k, amax, s);
        if (st != NVFP4_OK)
            return st;
    }
    return NVFP4_OK;
}

nvfp4_status nvfp4_fake_quant(const void* x, void* y, int64_t rows, int64_t cols,
                              const float* amax_in, float* amax_out, void* stream)
{
    int64_t n = 0;
    nvfp4_status st = check_matrix(rows, cols, &n);
    if (st != NVFP4_OK)
        return st;
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
        st = enqueue_amax_one(x, n, amax_out, s);
        if (st != NVFP4_OK)
            return st;
        a = amax_out;
    }
    if (n == 0)
        return NVFP4_OK;
    const int64_t nblocks = n / 16;
    k_fake_quant<<<persistent_grid(nblocks, (int64_t)kThreads * kUnroll, NVFP4_FQ_WG_PER_CU), kThreads, 0, s>>>(
        static_cast<const uint4*>(x), static_cast<uint4*>(y), nblocks, a);
    return launched();
}

nvfp4_status nvfp4_quantize_pack(const void* x, int64_t rows, int64_t cols,
                                 const float* amax_in, float* amax_out,
                                 uint8_t* packed, uint8_t* scales, float* global_scale,
                                 void* stream)
{
    int64_t n = 0;
    nvfp4_status st = check_matrix(rows, cols, &n);
    if (st != NVFP4_OK)
        return st;
    if ((n > 0 && (!x || !packed || !scales)) || !global_scale || (!amax_in && !amax_out))
        return NVFP4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(packed, 8) || !aligned(global_scale, 4) ||
        (amax_in && !aligned(amax_in, 4)) || (!amax_in && !aligned(amax_out, 4)))
        return NVFP4_ERR_ALIGN;
    const uint64_t xb = 2 * (uint64_t)n, pb = (uint64_t)n / 2, sb = (uint64_t)n / 16;
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
        st = enqueue_amax_one(x, n, amax_out, s);
        if (st != NVFP4_OK)
            return st;
        a = amax_out;
    }
    const int64_t nblocks = n / 16;
    k_quantize_pack<<<persistent_grid(nblocks, (int64_t)kThreads * kUnroll, NVFP4_QP_WG_PER_CU), kThreads, 0, s>>>(
        static_cast<const uint4*>(x), reinterpret_cast<uint2*>(packed), scales, global_scale,
        nblocks, a);
    return launched();
}

nvfp4_status nvfp4_dequant_unpack(const uint8_t* packed, const uint8_t* scales,
                                  const float* global_scale, int64_t rows, int64_t cols,
                                  void* y, void* stream)
{
    int64_t n = 0;
    nvfp4_status st = check_matrix(rows, cols, &n);
    if (st != NVFP4_OK)
        return st;
    if (n == 0)
        return NVFP4_OK;
    if (!packed || !scales || !global_scale || !y)
        return NVFP4_ERR_NULL;
    if (!aligned(packed, 8) || !aligned(y, 16) || !aligned(global_scale, 4))
        return NVFP4_ERR_ALIGN;
    const uint64_t yb = 2 * (uint64_t)n;
    if (overlap(y, yb, packed, (uint64_t)n / 2) || overlap(y, yb, scales, (uint64_t)n / 16) ||
        overlap(y, yb, global_scale, 4))
        return NVFP4_ERR_OVERLAP;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    const int64_t nblocks = n / 16;
    k_dequant_unpack<<<persistent_grid(nblocks, (int64_t)kThreads * kDqUnroll, NVFP4_DQ_WG_PER_CU), kThreads, 0, s>>>(
        reinterpret_cast<const uint2*>(packed), scales, global_scale, static_cast<uint4*>(y), nblocks);
    return launched();
}

nvfp4_status nvfp4_observer_update(float* state, const float* cur, int mode, float decay,
                                   void* stream)
{
    if (!state || !cur)
        return NVFP4_ERR_NULL;
    if (!aligned(state, 4) || !aligned(cur, 4))
        return NVFP4_ERR_ALIGN;
    if (mode != NVFP4_OBS_STATIC_MINMAX && mode != NVFP4_OBS_EMA)
        return NVFP4_ERR_ARG;
    if (mode == NVFP4_OBS_EMA && !(decay > 0.0f && decay <= 1.0f))
        return NVFP4_ERR_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    k_observer<<<1, 1, 0, s>>>(state, cur, mode, decay);
    return launched();
}

}  // extern "C"
