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
// * The per-tensor amax is a separate streaming pass with one atomic max per
//   workgroup; the quantizing kernels read it from device memory, so a fused
//   call never returns to the host.
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

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "nvfp4.h"

namespace {

// Launch shape and cache hints per kernel.  The defaults come from sweeps on
// MI355X (c5 weight, 470 MB); the macros let a build be re-tuned without
// editing the kernels.
#ifndef NVFP4_UNROLL
#define NVFP4_UNROLL 4            // half blocks per lane per iteration: fake-quant, pack
#endif
#ifndef NVFP4_DQ_UNROLL
#define NVFP4_DQ_UNROLL 8         // half blocks per lane per iteration: unpack
#endif
#ifndef NVFP4_AMAX_UNROLL
#define NVFP4_AMAX_UNROLL 4       // 16-byte vectors per lane per amax chunk
#endif
#ifndef NVFP4_AMAX_WG_PER_CU
#define NVFP4_AMAX_WG_PER_CU 2    // persistent workgroups per CU (each ends in one atomic)
#endif
#ifndef NVFP4_AMAX_PREFETCH
#define NVFP4_AMAX_PREFETCH 1     // 1: the amax loop loads chunk c + grid while folding chunk c
#endif
#ifndef NVFP4_FQ_WG_PER_CU
#define NVFP4_FQ_WG_PER_CU 64
#endif
#ifndef NVFP4_QP_WG_PER_CU
#define NVFP4_QP_WG_PER_CU 64
#endif
// Tensors below NVFP4_MID_BYTES get at most NVFP4_MID_WG_PER_CU quantizing
// workgroups per CU: each then covers several iterations (fewer table builds,
// loads of the next iteration in flight), 2-4 us faster on 64-112 MB tensors
// and slower on the 470 MB one.
#ifndef NVFP4_MID_BYTES
#define NVFP4_MID_BYTES (256LL << 20)
#endif
#ifndef NVFP4_MID_WG_PER_CU
#define NVFP4_MID_WG_PER_CU 8
#endif
// Partial maxima the workspace holds (one per amax workgroup), from byte 256.
#define NVFP4_MAX_PARTIALS ((NVFP4_WORKSPACE_BYTES - 256) / 4)
#ifndef NVFP4_LIN_DEPTH
#define NVFP4_LIN_DEPTH 2         // K steps of weight loads in flight per linear wave (even)
#endif
#ifndef NVFP4_LIN_SCALES_LDS
#define NVFP4_LIN_SCALES_LDS 1    // stage the linear workgroup's scale rows in LDS when they fit
#endif
#ifndef NVFP4_LIN_KS
#define NVFP4_LIN_KS 0            // K step of the linear kernel (128, 256); 0: by shape
#endif
#ifndef NVFP4_LIN_W
#define NVFP4_LIN_W 0             // waves per linear workgroup (4 or 8); 0: by shape
#endif
#ifndef NVFP4_LIN_NT
#define NVFP4_LIN_NT 0            // 16-row weight tiles per linear workgroup (1..8); 0: by shape
#endif
#ifndef NVFP4_LIN_TILED_M
#define NVFP4_LIN_TILED_M 65      // rows of x from which the linear layer uses the tiled kernel
#endif
#ifndef NVFP4_TILE_WAVES
#define NVFP4_TILE_WAVES 4        // waves per tiled-linear workgroup
#endif
#ifndef NVFP4_TILE_NW
#define NVFP4_TILE_NW 1           // 32-row weight tiles per tiled-linear wave
#endif
#ifndef NVFP4_TILE_MW
#define NVFP4_TILE_MW 4           // 32-row x tiles per tiled-linear workgroup
#endif
#ifndef NVFP4_TILE_MW_SMALL
#define NVFP4_TILE_MW_SMALL 2     // the same, up to NVFP4_TILE_SMALL_M rows of x
#endif
#ifndef NVFP4_TILE_SMALL_M
#define NVFP4_TILE_SMALL_M 128
#endif
#ifndef NVFP4_TILE_DEPTH
#define NVFP4_TILE_DEPTH 6        // K steps of weight loads in flight per tiled-linear wave (even)
#endif
#ifndef NVFP4_DQ_WG_PER_CU
#define NVFP4_DQ_WG_PER_CU 32
#endif
// 1: the quantizing passes walk the tensor from its end, so they start on the
// data the amax pass read last (measured no better than forward on MI355X).
#ifndef NVFP4_REVERSE
#define NVFP4_REVERSE 0
#endif
// Non-temporal (streaming) hints on loads (LD) and stores (ST).  The amax pass
// reads its last NVFP4_AMAX_ALLOC_BYTES with allocating loads: that part stays in
// the Infinity Cache (256 MB), where the quantizing pass over the same tensor
// finds it.  The quantizing passes stream x in and their outputs out.
#ifndef NVFP4_AMAX_ALLOC_BYTES
#define NVFP4_AMAX_ALLOC_BYTES (192LL << 20)  // bytes at the end of an amax pass read with allocating loads
#endif
// The same for the amax pass in front of a quantizing pass over a tensor below
// NVFP4_MID_BYTES: quantize-pack (QP) and fake-quant (FQ: also the dual, group
// and observe calls).  Measured on MI355X (warm loops, 0-256 MB swept): fake-
// quant, which writes as many bytes as it reads, gains most from finding all of
// x in the cache; quantize-pack was fastest with only the last 8-16 MB
// allocated (64 MB tensor: 28.6 -> 25.8 us; 112 MB: 42.0 -> 40.6 us), its amax
// pass then streaming like the rest.  Above NVFP4_MID_BYTES both keep 192 MB.
#ifndef NVFP4_QP_AMAX_ALLOC_MID
#define NVFP4_QP_AMAX_ALLOC_MID (16LL << 20)
#endif
#ifndef NVFP4_FQ_AMAX_ALLOC_MID
#define NVFP4_FQ_AMAX_ALLOC_MID NVFP4_AMAX_ALLOC_BYTES
#endif
#ifndef NVFP4_FQ_NT_LD
#define NVFP4_FQ_NT_LD 1
#endif
#ifndef NVFP4_FQ_NT_ST
#define NVFP4_FQ_NT_ST 1
#endif
#ifndef NVFP4_QP_NT_LD
#define NVFP4_QP_NT_LD 1
#endif
#ifndef NVFP4_QP_NT_ST
#define NVFP4_QP_NT_ST 1
#endif
#ifndef NVFP4_DQ_NT_ST
#define NVFP4_DQ_NT_ST 1
#endif

constexpr int kThreads = 256;                    // 4 waves of 64
constexpr int kUnroll = NVFP4_UNROLL;
constexpr int kDqUnroll = NVFP4_DQ_UNROLL;
constexpr int kAmaxUnroll = NVFP4_AMAX_UNROLL;
constexpr bool kReverse = NVFP4_REVERSE != 0;

constexpr float kEps = 1e-12f;    // clamp of the amax and of the block scale
constexpr float kGsNumerator = 2688.0f;  // E4M3 max 448 times E2M1 max 6

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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
__device__ __forceinline__ void store4(uint32_t* p, uint32_t v)
{
    if (NT)
        __builtin_nontemporal_store(v, p);
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

// E4M3 byte 0..0x7F (sign clear) -> value.  0x7F (NaN) never reaches here as a scale.
__device__ __forceinline__ float e4m3_decode(uint32_t s)
{
    return s >= 8u ? __uint_as_float((s << 20) + (120u << 23)) : (float)s * 0x1p-9f;
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
// Everything a block needs beyond its own data depends only on its E4M3 scale
// byte S (0..0x7E), so each workgroup tabulates it once, for all 128 bytes, in
// LDS.  Entry for S (8 dwords, 32 bytes):
//   [0]  r ~ 1 / sq (binary32 bits), the multiplier of the fast path; the sign
//        bit is set when the fast path is NOT exact under this S
//   [1]  sd = decode(S) / gs (binary32 bits), the factor of the outputs
//   [2]  t4 | t4<<16    [3] t6 | t6<<16    [4] (t2-t6) | (t2-t6)<<16
//   [5]  (t0-1) | (t0-1)<<16    [6] t7 | t5<<16    [7] t3 | t1<<16
// t_i (i = 1..7) is the smallest magnitude bit pattern whose E2M1 index is >= i;
// t0 the smallest whose quotient is nonzero.
//
// Fast path: q' = fl(x * r) goes through the gfx950 FP4 converter, which rounds
// a binary32 value to E2M1 with ties to even (checked on every binary32 input).
// q' can differ from the exact quotient fl(x / sq) in its last bits, and the
// code differs only if some bf16 magnitude lands on different sides of a
// decision boundary.  Both decisions are monotone in |x|, so comparing them at
// the two bf16 values around each exact threshold t_i settles it for every
// input; an S that fails (or whose t0 is not 1) keeps the threshold path.
constexpr int kEntryWords = 8;
constexpr uint32_t kNotFast = 0x80000000u;
// How far (in ulps) the table build looks for a multiplier that passes the
// check when 1 / sq does not.  With 1 / sq rounded, about 1% of (gs, S) pairs
// fail, and on some tensors those are the common scale bytes (a third of the
// blocks of the c4 activations); one ulp either way fixes all that do not sit
// on an exact tie, which no multiplier can fix.
constexpr int kMultiplierSteps = 2;

__device__ __forceinline__ float bf16_value(uint32_t bits) { return __uint_as_float(bits << 16); }

// Does the fast path pass boundary b (strictly, or at-or-above) for magnitude bits m?
__device__ __forceinline__ bool fast_passes(uint32_t m, float r, float b, bool strict)
{
    const float q = bf16_value(m) * r;
    return strict ? q > b : q >= b;
}

// The fast decision agrees with the exact threshold t for every bf16 input.
__device__ __forceinline__ bool fast_agrees(uint32_t t, float r, float b, bool strict)
{
    return fast_passes(t, r, b, strict) && !fast_passes(t - 1u, r, b, strict);
}

__device__ void build_entry(uint32_t s, float gs, uint32_t* dst)
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
    // The multiplier: 1 / sq rounded, or, when that one fails the check, the
    // nearest binary32 neighbour that passes it (up to kMultiplierSteps ulps
    // away; any multiplier that passes gives the exact codes).
    const uint32_t r0 = __float_as_uint(1.0f / sq);
    uint32_t r = r0;
    bool fast = false;
    for (int k = 0; t0 == 1u && !fast && k <= 2 * kMultiplierSteps; ++k) {
        r = r0 + (uint32_t)((k + 1) / 2 * ((k & 1) ? 1 : -1));      // 0, +1, -1, +2, -2, ...
        const float rf = __uint_as_float(r);
        fast = fast_agrees(t1, rf, 0.25f, true) && fast_agrees(t2, rf, 0.75f, false) &&
               fast_agrees(t3, rf, 1.25f, true) && fast_agrees(t4, rf, 1.75f, false) &&
               fast_agrees(t5, rf, 2.5f, true) && fast_agrees(t6, rf, 3.5f, false) &&
               fast_agrees(t7, rf, 5.0f, true);
    }
    dst[0] = (fast ? r : r0) | (fast ? 0u : kNotFast);
    dst[1] = __float_as_uint(sd);
    dst[2] = t4 * 0x10001u;
    dst[3] = t6 * 0x10001u;
    dst[4] = ((t2 - t6) & 0xFFFFu) * 0x10001u;
    dst[5] = (t0 - 1u) * 0x10001u;
    dst[6] = t7 | (t5 << 16);
    dst[7] = t3 | (t1 << 16);
}

// Threshold path: idx for the two magnitudes m (15-bit fields) of one dword,
// a three-step search over the seven sorted thresholds.
__device__ __forceinline__ uint32_t threshold_index(uint32_t m, const uint32_t* e)
{
    const uint32_t n4 = pk_top(pk_sub(m, e[2]));                // [m < t4]
    const uint32_t ta = pk_mad(n4, e[4], e[3]);                 // n4 ? t2 : t6
    const uint32_t na = pk_top(pk_sub(m, ta));
    const uint32_t j = pk_mad(n4, 0x00020002u, na);             // 0..3
    const uint32_t sel = pk_mad(j, 0x02020202u, 0x01000100u);   // bytes 2j, 2j+1 per half
    const uint32_t tb = __builtin_amdgcn_perm(e[7], e[6], sel); // t7, t5, t3, t1 by j
    const uint32_t nb = pk_top(pk_sub(m, tb));
    return pk_mad(j, 0x00020002u, nb) ^ 0x00070007u;           // 7 - (2j + nb)
}

// Codes of four bf16 pairs (8 elements) as one dword of nibbles, threshold path.
__device__ __forceinline__ uint32_t codes_threshold(const uint32_t* w, const uint32_t* e)
{
    uint32_t out = 0;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint32_t m = w[p] & 0x7FFF7FFFu;
        // sign when x < 0 and |x| >= t0 (the quotient does not underflow to zero)
        const uint32_t neg = w[p] & pk_sub(e[5], m) & 0x80008000u;
        const uint32_t c = threshold_index(m, e) | (neg >> 12);
        out |= ((c | (c >> 12)) & 0xFFu) << (8 * p);
    }
    return out;
}

// Codes of one bf16 pair into byte P of `out`, fast path (converter).
template <int P>
__device__ __forceinline__ uint32_t code_pair_fast(uint32_t out, uint32_t w, float r)
{
    const uint32_t m = w & 0x7FFF7FFFu;
    // -0.0 must give code 0 (its quotient is not below zero): clear the sign of
    // a zero magnitude; the packed add sets bit 15 of a half exactly when m != 0
    const uint32_t v = w & (w32(h2(m) + h2(0x7FFF7FFFu)) | 0x7FFF7FFFu);
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, __uint_as_float(v << 16) * r,
                                                    __uint_as_float(v & 0xFFFF0000u) * r, 1.0f, P);
}

// Codes of four bf16 pairs as one dword of nibbles, fast path.
__device__ __forceinline__ uint32_t codes_fast(const uint32_t* w, float r)
{
    uint32_t out = 0;
    out = code_pair_fast<0>(out, w[0], r);
    out = code_pair_fast<1>(out, w[1], r);
    out = code_pair_fast<2>(out, w[2], r);
    out = code_pair_fast<3>(out, w[3], r);
    return out;
}

// Two codes (byte P of `codes`, even element in the low nibble) -> two bf16
// outputs bf16(LUT[code] * sd).  The converter turns a code into its exact
// signed E2M1 value (checked for every byte), the product is one binary32
// rounding, and the bf16 pack conversion rounds to nearest even (checked for
// every binary32 input); -0 codes give -0 outputs.
template <int P>
__device__ __forceinline__ uint32_t decode_pair(uint32_t codes, float sd)
{
    const f32x2 m = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, P);
    const f32x2 v = {m.x * sd, m.y * sd};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Sixteen codes (two dwords of nibbles) -> sixteen bf16 outputs in two 16-byte stores.
template <bool NtStore>
__device__ __forceinline__ void decode_store(uint32_t c0, uint32_t c1, float sd, uint4* y, int64_t b)
{
    store16<NtStore>(y + 2 * b, make_uint4(decode_pair<0>(c0, sd), decode_pair<1>(c0, sd),
                                           decode_pair<2>(c0, sd), decode_pair<3>(c0, sd)));
    store16<NtStore>(y + 2 * b + 1, make_uint4(decode_pair<0>(c1, sd), decode_pair<1>(c1, sd),
                                               decode_pair<2>(c1, sd), decode_pair<3>(c1, sd)));
}

// E4M3 scale byte of a block whose largest magnitude has the bf16 bits bm.
__device__ __forceinline__ uint32_t scale_byte_of(uint32_t bm, float gs)
{
    // bamax / 6 without a divide: a bf16 value has 8 significant bits, so its
    // quotient by 3 never lies within 2^-52 (relative) of a binary32 rounding
    // mid-point, and rounding the binary64 product with 1/6 once more to
    // binary32 gives the correctly rounded quotient (checked for every bf16).
    const float sixth = (float)((double)bf16_value(bm) * (1.0 / 6.0));
    // binary32 -> E4M3 by the converter: round to nearest even below 448 (checked
    // for every non-negative binary32); above it the converter gives NaN bytes,
    // which the min turns into the saturated 0x7E
    const uint32_t s = __builtin_amdgcn_cvt_pk_fp8_f32(sixth * gs, 0.0f, 0, false) & 0xFFu;
    return s < 0x7Eu ? s : 0x7Eu;
}

// Scale byte of a block from its eight dwords (one lane holds the whole block).
__device__ __forceinline__ uint32_t block_scale_byte(const uint32_t (&w)[8], float gs)
{
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        mx = pk_max(mx, w[i] & 0x7FFF7FFFu);
    return scale_byte_of(max(mx & 0xFFFFu, mx >> 16), gs);
}

// ---------------------------------------------------------------- half blocks
//
// The streaming kernels give each lane half a block: lanes 2k and 2k+1 hold the
// two 8-element halves of one block, so every load and store is contiguous
// across the wave (16 bytes per lane of bf16, 4 bytes per lane of codes).  On
// MI355X this layout, with streaming (non-temporal) loads and stores, moves a
// read-and-write stream ~15% faster than one lane per block accessing 32
// bytes at a 32-byte lane stride.  The two lanes of a block are always both
// active or both inactive: element counts of whole-block tensors are even in
// halves, and every guard compares an even-aligned pair the same way.

// Largest magnitude (bf16 bits) of the block whose half this lane holds: its
// own four dwords, then the partner lane's maximum by a DPP quad permute
// [1, 0, 3, 2] (lane 2k <-> 2k+1).
__device__ __forceinline__ uint32_t pair_max(const uint32_t (&w)[4])
{
    const uint32_t mx = pk_max(pk_max(w[0] & 0x7FFF7FFFu, w[1] & 0x7FFF7FFFu),
                               pk_max(w[2] & 0x7FFF7FFFu, w[3] & 0x7FFF7FFFu));
    const uint32_t m = max(mx & 0xFFFFu, mx >> 16);
    return max(m, (uint32_t)__builtin_amdgcn_update_dpp((int)m, (int)m, 0xB1, 0xF, 0xF, false));
}

// The eight codes of four bf16 pairs (one dword of nibbles) under table entry e.
__device__ __forceinline__ uint32_t half_codes(const uint32_t* w, const uint32_t* e)
{
    const uint32_t head = e[0];
    if (!(head & kNotFast))
        return codes_fast(w, __uint_as_float(head));
    uint32_t t[6];
    const uint4 a = *reinterpret_cast<const uint4*>(e + 2);
    const uint2 b = *reinterpret_cast<const uint2*>(e + 6);
    t[0] = a.x; t[1] = a.y; t[2] = a.z; t[3] = a.w; t[4] = b.x; t[5] = b.y;
    return codes_threshold(w, t - 2);
}

// Eight codes -> eight bf16 outputs (16 bytes).
__device__ __forceinline__ uint4 decode_half(uint32_t c, float sd)
{
    return make_uint4(decode_pair<0>(c, sd), decode_pair<1>(c, sd), decode_pair<2>(c, sd),
                      decode_pair<3>(c, sd));
}

// Fake-quant of a half block whose block maximum is bm, into y[j].
template <bool NtStore>
__device__ __forceinline__ void fake_quant_half(const uint32_t (&w)[4], uint32_t bm, const uint32_t* tab,
                                                float gs, uint4* y, int64_t j)
{
    const uint32_t* e = tab + scale_byte_of(bm, gs) * kEntryWords;
    store16<NtStore>(y + j, decode_half(half_codes(w, e), __uint_as_float(e[1])));
}

// The 16 codes of a block (two dwords of nibbles) and its table entry.
__device__ __forceinline__ void block_codes(const uint32_t (&w)[8], const uint32_t* e, uint32_t& c0,
                                            uint32_t& c1)
{
    c0 = half_codes(w, e);
    c1 = half_codes(w + 4, e);
}

// Quantize-pack one block: eight code bytes into packed[b], its scale byte into scales[b].
template <bool NtStore>
__device__ __forceinline__ void pack_block(const uint32_t (&w)[8], const uint32_t* tab, float gs,
                                           uint2* packed, uint8_t* scales, int64_t b)
{
    const uint32_t s = block_scale_byte(w, gs);
    uint32_t c0, c1;
    block_codes(w, tab + s * kEntryWords, c0, c1);
    store8<NtStore>(packed + b, make_uint2(c0, c1));
    scales[b] = (uint8_t)s;
}

// Workgroup max of the lanes' packed maxima (15-bit magnitude); valid in thread 0.
__device__ __forceinline__ uint32_t workgroup_max(uint32_t mx, uint32_t* wave_max)
{
    uint32_t m = max(mx & 0xFFFFu, mx >> 16);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
    if ((threadIdx.x & 63) == 0)
        wave_max[threadIdx.x >> 6] = m;
    __syncthreads();
    uint32_t r = wave_max[0];
#pragma unroll
    for (int i = 1; i < kThreads / 64; ++i)
        r = max(r, wave_max[i]);
    return r;
}

// ---------------------------------------------------------------- kernels

// i-th unit (half block, or block for the ragged kernels) of a pass, or -1 past
// the end; the pass runs backwards when kReverse.
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
    int64_t alloc_from;                            // chunks from here on load into the caches
    const float* snap_from[2];                     // workgroup 0 copies *snap_from[i] to snap_to[i],
    float* snap_to;                                // i < nsnap (observer states before their step)
    int32_t nsnap;
};

// max |x| over a group of tensors.  Atomic mode: one signed-integer atomic max
// per workgroup on the fp32 bits of the result (non-negative floats order like
// their bits, and a negative prior value loses to any of them).  Partials mode
// (the workspace calls): workgroup i stores its maximum in partials[i] instead
// and k_amax_finish reduces them, so no launch clears the amax first and no
// atomics contend at the end of the pass.
template <bool Partials>
__global__ __launch_bounds__(kThreads) void k_amax(AmaxGroup g, float* out, uint32_t* partials)
{
    constexpr int64_t kChunk = (int64_t)kThreads * kAmaxUnroll;
    if (blockIdx.x == 0 && threadIdx.x == 0)
        for (int i = 0; i < g.nsnap; ++i)
            g.snap_to[i] = *g.snap_from[i];
    uint32_t mx = 0;
    const int64_t total = g.chunk_end[g.count - 1];
    // chunks only grow along the loop, so the current tensor is cached and
    // advanced instead of searched for on every chunk
    int t = 0;
    int64_t begin = 0, end = g.chunk_end[0], n = g.nvec[0];
    const uint4* __restrict__ src = g.vec[0];
    // the vectors of chunk c (zeros past the end of its tensor)
    auto load_chunk = [&](int64_t c, uint4 (&v)[kAmaxUnroll]) {
        while (c >= end) {
            ++t;
            begin = end;
            end = g.chunk_end[t];
            n = g.nvec[t];
            src = g.vec[t];
        }
        const int64_t first = (c - begin) * kChunk + threadIdx.x;
#pragma unroll
        for (int u = 0; u < kAmaxUnroll; ++u) {
            const int64_t i = first + (int64_t)u * kThreads;
            v[u] = i >= n                ? make_uint4(0u, 0u, 0u, 0u)
                   : c >= g.alloc_from ? load16<false>(src + i)
                                       : load16<true>(src + i);
        }
    };
    auto fold = [&](const uint4 (&v)[kAmaxUnroll]) {
#pragma unroll
        for (int u = 0; u < kAmaxUnroll; ++u) {
            mx = pk_max(mx, v[u].x & 0x7FFF7FFFu);
            mx = pk_max(mx, v[u].y & 0x7FFF7FFFu);
            mx = pk_max(mx, v[u].z & 0x7FFF7FFFu);
            mx = pk_max(mx, v[u].w & 0x7FFF7FFFu);
        }
    };
    if (NVFP4_AMAX_PREFETCH) {
        // the next chunk's loads are in flight while the current one is folded
        uint4 cur[kAmaxUnroll], nxt[kAmaxUnroll];
        int64_t c = blockIdx.x;
        if (c < total)
            load_chunk(c, cur);
        for (; c < total; c += gridDim.x) {
            if (c + gridDim.x < total)
                load_chunk(c + gridDim.x, nxt);
            fold(cur);
#pragma unroll
            for (int u = 0; u < kAmaxUnroll; ++u)
                cur[u] = nxt[u];
        }
    } else {
        for (int64_t c = blockIdx.x; c < total; c += gridDim.x) {
            uint4 v[kAmaxUnroll];
            load_chunk(c, v);
            fold(v);
        }
    }
    if (blockIdx.x == 0) {
        for (int t = 0; t < g.count; ++t)
            if ((int)threadIdx.x < g.ntail[t])
                mx = pk_max(mx, g.tail[t][threadIdx.x] & 0x7FFFu);
    }
    __shared__ uint32_t wave_max[kThreads / 64];
    const uint32_t r = workgroup_max(mx, wave_max);
    if (Partials) {
        if (threadIdx.x == 0)
            partials[blockIdx.x] = r;
        return;
    }
    if (threadIdx.x == 0) {
        // Same-address atomics serialise at the coherence point; the maximum only
        // grows, so a workgroup that already sees a value at least as large as its
        // own has nothing to add (a stale read costs one redundant atomic at most).
        int* dst = reinterpret_cast<int*>(out);
        const int mine = (int)(r << 16);
        if (mine > __hip_atomic_load(dst, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            atomicMax(dst, mine);
    }
}

// The kUnroll half blocks of one iteration of a quantizing pass (zeros past the end).
template <bool NtLd>
__device__ __forceinline__ void load_halves(const uint4* x, int64_t base, int64_t nhalves,
                                            uint4 (&v)[kUnroll])
{
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const int64_t j = walk(base + (int64_t)u * kThreads, nhalves);
        v[u] = j >= 0 ? load16<NtLd>(x + j) : make_uint4(0u, 0u, 0u, 0u);
    }
}

// A quantizing pass over all half blocks with a grid stride; body(w, j) gets
// the four dwords of half j.  The first iteration's loads are issued before
// the workgroup builds its scale-byte table, so the table build hides under
// their latency.
// With Fence, the loads issued before the pass (the partial maxima) stay ahead
// of the loads of x, so build() waits for them alone.
template <bool NtLd, bool Fence, typename Build, typename Body>
__device__ __forceinline__ void quantize_pass(const uint4* x, int64_t nhalves, Build build,
                                              Body body)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads * kUnroll;
    int64_t base = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x;
    uint4 v[kUnroll];
    if (Fence)
        __builtin_amdgcn_sched_barrier(0);
    load_halves<NtLd>(x, base, nhalves, v);
    build();
    __syncthreads();
    for (; base < nhalves; base += stride) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t j = walk(base + (int64_t)u * kThreads, nhalves);
            if (j >= 0) {
                const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
                body(w, j);
            }
        }
        load_halves<NtLd>(x, base + stride, nhalves, v);
    }
}

// Observer states of up to two observers (verl QATLinear page, section 5).
struct ObserverArgs {
    float* state[2];
    int mode[2];
    float decay[2];
};

// One observer step: the new state from state s and the step amax c.
__device__ __forceinline__ float observer_value(float s, float c, int mode, float decay)
{
    if (s < 0.0f)
        return c;                                  // first observation
    if (mode == NVFP4_OBS_STATIC_MINMAX)
        return c > s ? c : s;
    const float keep = 1.0f - decay;
    const float a = keep * s;
    const float b = decay * c;
    return a + b;                                  // no contraction: -ffp-contract=off
}

// Observer steps of up to two states on the same step amax c, in place.
__device__ void observer_steps(float c, const ObserverArgs& o, int n)
{
    for (int i = 0; i < n; ++i)
        *o.state[i] = observer_value(*o.state[i], c, o.mode[i], o.decay[i]);
}

// Where a quantizing pass takes its amax from: amax[0] (and amax[1] for the dual
// pass), or (workspace calls) the partial maxima of the amax pass, which every
// workgroup reduces itself, so no launch sits between the two passes.  From
// the partials, the pass quantizes with the reduced amax c, or, with nobs
// observers, with their new states observer(prior[i], c); prior holds the
// states as the amax pass copied them, so workgroup 0 may store the new states
// (and c in *store) while other workgroups have yet to start.
struct AmaxIn {
    const float* amax[2];
    const uint32_t* partials;     // 16-byte aligned, at most NVFP4_MAX_PARTIALS
    int count;
    float* store;                 // may be null
    ObserverArgs obs;
    int nobs;
    const float* prior;
};

// Each lane's share of the partials: kPartialsPerLane consecutive slots (slots
// at or past count read as 0).  Vector loads, issued by every wave.
constexpr int kPartialsPerLane = NVFP4_MAX_PARTIALS / 64;
static_assert(NVFP4_MAX_PARTIALS % 256 == 0, "whole 16-byte loads of partials per lane");

struct PartialLoads {
    uint4 v[kPartialsPerLane / 4];
    float prior[2];
};

__device__ __forceinline__ PartialLoads load_partials(const AmaxIn& src)
{
    PartialLoads p;
    const int i = kPartialsPerLane * (int)(threadIdx.x & 63u);
    const uint4* q = reinterpret_cast<const uint4*>(src.partials + i);
#pragma unroll
    for (int k = 0; k < kPartialsPerLane / 4; ++k)
        p.v[k] = i < src.count ? q[k] : make_uint4(0u, 0u, 0u, 0u);
    p.prior[0] = src.nobs > 0 ? src.prior[0] : 0.0f;
    p.prior[1] = src.nobs > 1 ? src.prior[1] : 0.0f;
    return p;
}

// The amaxes the pass quantizes with, from the loaded partials: a max over the
// lane's valid slots, then across the wave (every wave computes it, so no
// barrier is needed), then the observer steps.
__device__ __forceinline__ void resolve_amax(const PartialLoads& p, const AmaxIn& src, float (&a)[2])
{
    const int i = kPartialsPerLane * (int)(threadIdx.x & 63u);
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < kPartialsPerLane / 4; ++k) {
        const uint32_t w[4] = {p.v[k].x, p.v[k].y, p.v[k].z, p.v[k].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
            m = i + 4 * k + e < src.count ? max(m, w[e]) : m;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
    const float c = __uint_as_float(m << 16);
    a[0] = src.nobs > 0 ? observer_value(p.prior[0], c, src.obs.mode[0], src.obs.decay[0]) : c;
    a[1] = src.nobs > 1 ? observer_value(p.prior[1], c, src.obs.mode[1], src.obs.decay[1]) : c;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (src.store)
            *src.store = c;
        if (src.nobs > 0)
            *src.obs.state[0] = a[0];
        if (src.nobs > 1)
            *src.obs.state[1] = a[1];
    }
}

// The amax of a single-amax pass: issue the loads it needs (before the loads
// of x), then finish it once they are in.  Without partials the pass reads
// *src.amax[0] directly, and no fence orders that load against the loads of x.
template <bool Partials>
struct AmaxOfPass {
    PartialLoads p;
    float direct;

    __device__ __forceinline__ explicit AmaxOfPass(const AmaxIn& src)
    {
        if (Partials)
            p = load_partials(src);
        else
            direct = *src.amax[0];
    }
    __device__ __forceinline__ float finish(const AmaxIn& src) const
    {
        if (!Partials)
            return direct;
        float a[2];
        resolve_amax(p, src, a);
        return a[0];
    }
};

// Threads 0..127 tabulate the 128 scale bytes under gs (the other threads idle).
__device__ __forceinline__ void build_table(float gs, uint32_t* tab)
{
    if (threadIdx.x < 128)
        build_entry(threadIdx.x, gs, tab + threadIdx.x * kEntryWords);
}

template <bool Partials>
__global__ __launch_bounds__(kThreads) void k_fake_quant(const uint4* x, uint4* y,
                                                         int64_t nhalves, AmaxIn src)
{
    __shared__ uint4 table[128 * kEntryWords / 4];
    uint32_t* tab = reinterpret_cast<uint32_t*>(table);
    const AmaxOfPass<Partials> am(src);
    float gs = Partials ? 0.0f : global_scale_of(am.direct);
    quantize_pass<NVFP4_FQ_NT_LD != 0, Partials>(x, nhalves, [&] {
        if (Partials)
            gs = global_scale_of(am.finish(src));
        build_table(gs, tab);
    }, [&](const uint32_t (&w)[4], int64_t j) {
        fake_quant_half<NVFP4_FQ_NT_ST != 0>(w, pair_max(w), tab, gs, y, j);
    });
}

// One read of x, fake-quantized under two amaxes into y0 and y1: an activation
// seen by two observers (verl QATLinear page, section 5) costs 2 + 2 * 2 bytes
// per element instead of 2 * (2 + 2).  Each half of the workgroup tabulates
// one amax.  A lane reads its half block before writing either output, so
// y0 == x or y1 == x (in place) is safe.
static_assert(kThreads == 256, "the dual table build gives each amax 128 threads");
template <bool Partials>
__global__ __launch_bounds__(kThreads) void k_fake_quant_dual(const uint4* x, uint4* y0,
                                                              uint4* y1, int64_t nhalves, AmaxIn src)
{
    __shared__ uint4 table[2 * 128 * kEntryWords / 4];
    uint32_t* tab = reinterpret_cast<uint32_t*>(table);
    PartialLoads p;
    float gs0 = 0.0f, gs1 = 0.0f;
    if (Partials) {
        p = load_partials(src);
    } else {
        gs0 = global_scale_of(*src.amax[0]);
        gs1 = global_scale_of(*src.amax[1]);
    }
    quantize_pass<NVFP4_FQ_NT_LD != 0, Partials>(x, nhalves, [&] {
        if (Partials) {
            float a[2];
            resolve_amax(p, src, a);
            gs0 = global_scale_of(a[0]);
            gs1 = global_scale_of(a[1]);
        }
        const uint32_t half = threadIdx.x >> 7, s = threadIdx.x & 127u;
        build_entry(s, half ? gs1 : gs0, tab + (half * 128u + s) * kEntryWords);
    }, [&](const uint32_t (&w)[4], int64_t j) {
        const uint32_t bm = pair_max(w);
        fake_quant_half<NVFP4_FQ_NT_ST != 0>(w, bm, tab, gs0, y0, j);
        fake_quant_half<NVFP4_FQ_NT_ST != 0>(w, bm, tab + 128 * kEntryWords, gs1, y1, j);
    });
}

// Tensors that share one amax (fused siblings, verl QATLinear page, section 4),
// fake-quantized in one launch.  Their half blocks are visited in chunks of
// kThreads * kUnroll, one chunk per workgroup iteration as in quantize_pass; a
// chunk never spans two tensors, so the tensor of a chunk is the same for the
// whole workgroup and its pointers stay scalar.
struct FqGroup {
    const uint4* x[NVFP4_AMAX_GROUP_MAX];
    uint4* y[NVFP4_AMAX_GROUP_MAX];
    int64_t nhalves[NVFP4_AMAX_GROUP_MAX];
    int64_t chunk_end[NVFP4_AMAX_GROUP_MAX];    // running sum of ceil(nhalves / chunk)
    int32_t count;
};

template <bool Partials>
__global__ __launch_bounds__(kThreads) void k_fake_quant_group(FqGroup g, AmaxIn src)
{
    constexpr int64_t kChunk = (int64_t)kThreads * kUnroll;
    __shared__ uint4 table[128 * kEntryWords / 4];
    uint32_t* tab = reinterpret_cast<uint32_t*>(table);
    const AmaxOfPass<Partials> am(src);
    float gs = Partials ? 0.0f : global_scale_of(am.direct);
    if (Partials)
        __builtin_amdgcn_sched_barrier(0);
    const int64_t total = g.chunk_end[g.count - 1];
    // chunks only grow along the loop, so the tensor cursor only moves forward
    int t = 0;
    int64_t begin = 0;
    auto seek = [&](int64_t c) {
        while (c >= g.chunk_end[t]) {
            begin = g.chunk_end[t];
            ++t;
        }
    };
    int64_t c = blockIdx.x;
    uint4 v[kUnroll];
    if (c < total) {
        seek(c);
        load_halves<NVFP4_FQ_NT_LD != 0>(g.x[t], (c - begin) * kChunk + threadIdx.x, g.nhalves[t], v);
    }
    if (Partials)
        gs = global_scale_of(am.finish(src));
    build_table(gs, tab);
    __syncthreads();
    for (; c < total; c += gridDim.x) {
        const int64_t base = (c - begin) * kChunk + threadIdx.x, n = g.nhalves[t];
        uint4* y = g.y[t];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t j = walk(base + (int64_t)u * kThreads, n);
            if (j >= 0) {
                const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
                fake_quant_half<NVFP4_FQ_NT_ST != 0>(w, pair_max(w), tab, gs, y, j);
            }
        }
        if (c + gridDim.x < total) {
            seek(c + gridDim.x);
            load_halves<NVFP4_FQ_NT_LD != 0>(g.x[t], (c + gridDim.x - begin) * kChunk + threadIdx.x,
                                             g.nhalves[t], v);
        }
    }
}

// Quantize-pack: lane j stores the eight codes of half j (one dword of the
// packed codes); the even lane of a block also stores its scale byte.
template <bool Partials>
__global__ __launch_bounds__(kThreads) void k_quantize_pack(const uint4* __restrict__ x,
                                                            uint32_t* __restrict__ packed,
                                                            uint8_t* __restrict__ scales,
                                                            float* __restrict__ gs_out,
                                                            int64_t nhalves, AmaxIn src)
{
    __shared__ uint4 table[128 * kEntryWords / 4];
    uint32_t* tab = reinterpret_cast<uint32_t*>(table);
    const AmaxOfPass<Partials> am(src);
    float gs = Partials ? 0.0f : global_scale_of(am.direct);
    if (!Partials && blockIdx.x == 0 && threadIdx.x == 0)
        *gs_out = gs;
    quantize_pass<NVFP4_QP_NT_LD != 0, Partials>(x, nhalves, [&] {
        if (Partials) {
            gs = global_scale_of(am.finish(src));
            if (blockIdx.x == 0 && threadIdx.x == 0)
                *gs_out = gs;
        }
        build_table(gs, tab);
    }, [&](const uint32_t (&w)[4], int64_t j) {
        const uint32_t sb = scale_byte_of(pair_max(w), gs);
        store4<NVFP4_QP_NT_ST != 0>(packed + j, half_codes(w, tab + sb * kEntryWords));
        if (!(j & 1))
            scales[j >> 1] = (uint8_t)sb;
    });
}

// Two lanes per block: lane j decodes the eight codes of dword j of the packed
// codes (half j % 2 of block j / 2) with that block's scale byte and writes its
// eight bf16 outputs, 16 bytes at j.  Every stream is then contiguous across a
// wave (4-byte code loads, 16-byte stores), which writes the output ~20% faster
// on MI355X than one lane per block storing 32 bytes at a 32-byte lane stride.
__global__ __launch_bounds__(kThreads) void k_dequant_unpack(const uint32_t* __restrict__ packed,
                                                             const uint8_t* __restrict__ scales,
                                                             const float* __restrict__ gs_in,
                                                             uint4* __restrict__ y, int64_t nhalves)
{
    __shared__ float sd_of[128];                   // decode(S) / gs for every scale byte
    const float gs = *gs_in;
    if (threadIdx.x < 128)
        sd_of[threadIdx.x] = e4m3_decode(threadIdx.x) / gs;
    __syncthreads();

    // software-pipelined: the next iteration's codes and scales are in flight
    // while the current ones are decoded and stored
    const int64_t stride = (int64_t)gridDim.x * kThreads * kDqUnroll;
    int64_t base = (int64_t)blockIdx.x * kThreads * kDqUnroll + threadIdx.x;
    uint32_t p[kDqUnroll], s[kDqUnroll];
#pragma unroll
    for (int u = 0; u < kDqUnroll; ++u) {
        const int64_t j = base + (int64_t)u * kThreads;
        p[u] = j < nhalves ? packed[j] : 0u;
        s[u] = j < nhalves ? scales[j >> 1] : 0u;
    }
    for (; base < nhalves; base += stride) {
        uint32_t pn[kDqUnroll], sn[kDqUnroll];
#pragma unroll
        for (int u = 0; u < kDqUnroll; ++u) {
            const int64_t j = base + stride + (int64_t)u * kThreads;
            pn[u] = j < nhalves ? packed[j] : 0u;
            sn[u] = j < nhalves ? scales[j >> 1] : 0u;
        }
#pragma unroll
        for (int u = 0; u < kDqUnroll; ++u) {
            const int64_t j = base + (int64_t)u * kThreads;
            if (j < nhalves) {
                const float sd = sd_of[s[u] & 0x7Fu];
                store16<NVFP4_DQ_NT_ST != 0>(y + j, make_uint4(decode_pair<0>(p[u], sd), decode_pair<1>(p[u], sd),
                                                               decode_pair<2>(p[u], sd), decode_pair<3>(p[u], sd)));
            }
        }
#pragma unroll
        for (int u = 0; u < kDqUnroll; ++u) {
            p[u] = pn[u];
            s[u] = sn[u];
        }
    }
}

// ---------------------------------------------------------------- ragged rows
//
// A row whose length is not a multiple of 16 is zero-padded to the next
// multiple (VideoX-Fun page, quantize_weight_to_float4): its last block holds
// fewer than 16 elements and zeros, which never change a block max.  Packed
// codes and scales keep the padded layout ([rows, 8 * nbr] and [rows, nbr] for
// nbr = ceil(cols / 16)), so block f is still byte 8f and scale f; only the
// bf16 side is addressed per element.  Rows may start at any element, so the
// half-block layout's vector accesses do not apply: one lane owns one block.
struct RaggedShape {
    int64_t cols;       // elements per row
    int64_t nbr;        // blocks per row
    int64_t nblocks;    // rows * nbr
};

// First element and element count of block f.
__device__ __forceinline__ int64_t ragged_block(const RaggedShape& g, int64_t f, int& n)
{
    const int64_t r = f / g.nbr;
    const int64_t c0 = (f - r * g.nbr) * 16;
    const int64_t left = g.cols - c0;
    n = left < 16 ? (int)left : 16;
    return r * g.cols + c0;
}

__device__ __forceinline__ void load_ragged(const uint16_t* x, int64_t e0, int n,
                                            uint32_t (&w)[8])
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t lo = 2 * i < n ? x[e0 + 2 * i] : 0u;
        const uint32_t hi = 2 * i + 1 < n ? x[e0 + 2 * i + 1] : 0u;
        w[i] = lo | (hi << 16);
    }
}

__device__ __forceinline__ void store_ragged(uint16_t* y, int64_t e0, int n, uint32_t c0, uint32_t c1,
                                             float sd)
{
    const uint32_t o[8] = {decode_pair<0>(c0, sd), decode_pair<1>(c0, sd), decode_pair<2>(c0, sd),
                           decode_pair<3>(c0, sd), decode_pair<0>(c1, sd), decode_pair<1>(c1, sd),
                           decode_pair<2>(c1, sd), decode_pair<3>(c1, sd)};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (2 * i < n)
            y[e0 + 2 * i] = (uint16_t)(o[i] & 0xFFFFu);
        if (2 * i + 1 < n)
            y[e0 + 2 * i + 1] = (uint16_t)(o[i] >> 16);
    }
}

__global__ __launch_bounds__(kThreads) void k_fake_quant_ragged(const uint16_t* x,
                                                                uint16_t* y, RaggedShape g,
                                                                const float* __restrict__ amax)
{
    __shared__ uint4 table[128 * kEntryWords / 4];
    uint32_t* tab = reinterpret_cast<uint32_t*>(table);
    const float gs = global_scale_of(*amax);
    if (threadIdx.x < 128)
        build_entry(threadIdx.x, gs, tab + threadIdx.x * kEntryWords);
    __syncthreads();
    for (int64_t f = (int64_t)blockIdx.x * kThreads + threadIdx.x; f < g.nblocks;
         f += (int64_t)gridDim.x * kThreads) {
        int n;
        const int64_t e0 = ragged_block(g, f, n);
        uint32_t w[8];
        load_ragged(x, e0, n, w);
        const uint32_t* e = tab + block_scale_byte(w, gs) * kEntryWords;
        uint32_t c0, c1;
        block_codes(w, e, c0, c1);
        store_ragged(y, e0, n, c0, c1, __uint_as_float(e[1]));
    }
}

__global__ __launch_bounds__(kThreads) void k_quantize_pack_ragged(const uint16_t* __restrict__ x,
                                                                   uint2* __restrict__ packed,
                                                                   uint8_t* __restrict__ scales,
                                                                   float* __restrict__ gs_out,
                                                                   RaggedShape g,
                                                                   const float* __restrict__ amax)
{
    __shared__ uint4 table[128 * kEntryWords / 4];
    uint32_t* tab = reinterpret_cast<uint32_t*>(table);
    const float gs = global_scale_of(*amax);
    if (threadIdx.x < 128)
        build_entry(threadIdx.x, gs, tab + threadIdx.x * kEntryWords);
    if (blockIdx.x == 0 && threadIdx.x == 0)
        *gs_out = gs;
    __syncthreads();
    for (int64_t f = (int64_t)blockIdx.x * kThreads + threadIdx.x; f < g.nblocks;
         f += (int64_t)gridDim.x * kThreads) {
        int n;
        const int64_t e0 = ragged_block(g, f, n);
        uint32_t w[8];
        load_ragged(x, e0, n, w);
        pack_block<false>(w, tab, gs, packed, scales, f);
    }
}

__global__ __launch_bounds__(kThreads) void k_dequant_unpack_ragged(const uint2* __restrict__ packed,
                                                                    const uint8_t* __restrict__ scales,
                                                                    const float* __restrict__ gs_in,
                                                                    uint16_t* __restrict__ y,
                                                                    RaggedShape g)
{
    const float gs = *gs_in;
    for (int64_t f = (int64_t)blockIdx.x * kThreads + threadIdx.x; f < g.nblocks;
         f += (int64_t)gridDim.x * kThreads) {
        int n;
        const int64_t e0 = ragged_block(g, f, n);
        const uint2 p = packed[f];
        store_ragged(y, e0, n, p.x, p.y, e4m3_decode(scales[f] & 0x7Fu) / gs);
    }
}

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
    f32x4 (*partial)[MT * NT][64] = reinterpret_cast<f32x4 (*)[MT * NT][64]>(lin_lds);
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
    // (through the LDS the scales used, once every wave is past the K loop)
    if (SL)
        __syncthreads();
    if (wave > 0) {
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int t = 0; t < NT; ++t)
                partial[wave - 1][i * NT + t][lane] = acc[i][t];
    }
    __syncthreads();
    if (wave != 0)
        return;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            f32x4 v = acc[i][t];
#pragma unroll
            for (int w = 0; w < W - 1; ++w)
                v += partial[w][i * NT + t][lane];
            const int64_t n = n0 + 16 * t + r;
            if (n >= N)
                continue;
            const float b = bias ? bf16_value(bias[n]) : 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t m = m0 + 16 * i + 4 * g + e;
                if (m < M) {
                    const f32x2 o = {v[e] + b, 0.0f};
                    y[m * N + n] = (uint16_t)(__builtin_bit_cast(uint32_t, __builtin_convertvector(o, bf16x2)) & 0xFFFFu);
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
    const int64_t m0 = (int64_t)blockIdx.x * kRows;
    const int64_t n0 = ((int64_t)blockIdx.y * kTileWaves + wave) * 32 * NW;
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

__global__ void k_observer(const float* cur, ObserverArgs o, int n)
{
    observer_steps(*cur, o, n);
}

// The amax from the partial maxima (bf16 magnitude bits) of the amax pass, then
// n observer steps on it (n = 0: none).
__global__ __launch_bounds__(kThreads) void k_amax_finish(const uint32_t* partials, int count, float* amax,
                                                          ObserverArgs o, int n)
{
    uint32_t m = 0;
    for (int i = threadIdx.x; i < count; i += kThreads)
        m = max(m, partials[i]);
    __shared__ uint32_t wave_max[kThreads / 64];
    const uint32_t r = workgroup_max(m, wave_max);
    if (threadIdx.x == 0) {
        const float v = __uint_as_float(r << 16);
        *amax = v;
        observer_steps(v, o, n);
    }
}

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
int quant_wg_per_cu(int64_t nhalves, int large)
{
    return nhalves * 16 < NVFP4_MID_BYTES ? NVFP4_MID_WG_PER_CU : large;
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
    const float* a = src.amax[0];                  // the ragged kernels take a direct amax
    if (m.ragged) {
        const RaggedShape g{cols, m.nbr, m.nblocks};
        k_fake_quant_ragged<<<persistent_grid(m.nblocks, kThreads, kRaggedWgPerCu), kThreads, 0, s>>>(
            static_cast<const uint16_t*>(x), static_cast<uint16_t*>(y), g, a);
        return launched();
    }
    const int64_t nh = 2 * m.nblocks;
    const dim3 grid(persistent_grid(nh, (int64_t)kThreads * kUnroll, quant_wg_per_cu(nh, NVFP4_FQ_WG_PER_CU)));
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
    const float* a = src.amax[0];                  // the ragged kernel takes a direct amax
    if (m.ragged) {
        const RaggedShape g{cols, m.nbr, m.nblocks};
        k_quantize_pack_ragged<<<persistent_grid(m.nblocks, kThreads, kRaggedWgPerCu), kThreads, 0, s>>>(
            static_cast<const uint16_t*>(x), reinterpret_cast<uint2*>(packed), scales, global_scale, g, a);
        return launched();
    }
    const int64_t nh = 2 * m.nblocks;
    const dim3 grid(persistent_grid(nh, (int64_t)kThreads * kUnroll, quant_wg_per_cu(nh, NVFP4_QP_WG_PER_CU)));
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
        const dim3 grid(persistent_grid(chunks, 1, quant_wg_per_cu(chunks * kChunk, NVFP4_FQ_WG_PER_CU)));
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
    const size_t partial_bytes = (size_t)(W - 1) * MT * NT * 64 * sizeof(f32x4);
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
// x on the c5 weight), else 4 (the partial sums of 8 waves of several x tiles do
// not fit in LDS, and 16 waves spill registers).
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
    k_fake_quant_dual<false><<<persistent_grid(nh, (int64_t)kThreads * kUnroll,
                                               quant_wg_per_cu(nh, NVFP4_FQ_WG_PER_CU)),
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
    const nvfp4_status st = check_matrix(rows, cols, &m);
    if (st != NVFP4_OK)
        return st;
    if ((m.numel > 0 && (!x || !y)) || !workspace)
        return NVFP4_ERR_NULL;
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(workspace, 256) || (amax_out && !aligned(amax_out, 4)))
        return NVFP4_ERR_ALIGN;
    const uint64_t bytes = 2 * (uint64_t)m.numel;
    const Region in[1] = {{x, bytes}};
    const Region out[3] = {{y, bytes}, {amax_out, amax_out ? 4u : 0u}, {workspace, NVFP4_WORKSPACE_BYTES}};
    if (check_regions(in, 1, out, 3, true) != NVFP4_OK)
        return NVFP4_ERR_OVERLAP;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (m.numel == 0)
        return amax_out ? enqueue_reset(amax_out, s) : NVFP4_OK;
    if (!m.ragged) {
        // the pass reduces the partials itself and stores the amax
        AmaxIn src;
        if (enqueue_amax_partials(&x, &m.numel, 1, workspace, s, &src, ObserverArgs{}, 0,
                                  amax_alloc_bytes(2 * m.numel, NVFP4_FQ_AMAX_ALLOC_MID)) != NVFP4_OK)
            return NVFP4_ERR_HIP;
        src.store = amax_out;
        return enqueue_fake_quant(x, y, cols, m, src, s);
    }
    float* a = ws_amax(workspace, amax_out);
    if (enqueue_amax_ws(&x, &m.numel, 1, workspace, a, s) != NVFP4_OK)
        return NVFP4_ERR_HIP;
    return enqueue_fake_quant(x, y, cols, m, a, s);
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
    if (!m.ragged) {
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
    const unsigned grid = persistent_grid(nh, (int64_t)kThreads * kUnroll, quant_wg_per_cu(nh, NVFP4_FQ_WG_PER_CU));
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
    constexpr int kNW = NVFP4_TILE_NW;
    if (m < NVFP4_LIN_TILED_M || (n + 32 * kNW * kTileWaves - 1) / (32 * kNW * kTileWaves) > 65535)
        return enqueue_linear_mt<4>(x, m, k, packed, scales, global_scale, n, bias, y, s);
    if (m <= NVFP4_TILE_SMALL_M)
        return enqueue_linear_tiled<NVFP4_TILE_MW_SMALL, kNW>(x, m, k, packed, scales, global_scale, n, bias, y, s);
    return enqueue_linear_tiled<NVFP4_TILE_MW, kNW>(x, m, k, packed, scales, global_scale, n, bias, y, s);
}

}  // extern "C"
