// Device helpers of libnvfp4: packed 16-bit arithmetic, memory hints, the scalar
// number formats, the per-scale-byte table and the half-block codes and outputs
// (included by nvfp4.hip).

#ifndef NVFP4_DEVICE_HPP
#define NVFP4_DEVICE_HPP

#include <hip/hip_runtime.h>

#include "config.hpp"

namespace {

// ---------------------------------------------------------------- packed 16-bit helpers

__device__ __forceinline__ u16x2 h2(uint32_t v) { return __builtin_bit_cast(u16x2, v); }
__device__ __forceinline__ uint32_t w32(u16x2 v) { return __builtin_bit_cast(uint32_t, v); }

__device__ __forceinline__ uint32_t pk_max(uint32_t a, uint32_t b)
{
    return w32(__builtin_elementwise_max(h2(a), h2(b)));
}
__device__ __forceinline__ uint32_t pk_min(uint32_t a, uint32_t b)
{
    return w32(__builtin_elementwise_min(h2(a), h2(b)));
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
    return kGsNumerator / a;          // IEEE binary32 divide (compiled without fast-math)
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

// fl(v / sq) without a divide per element, from r = fl(1 / sq) (the correctly
// rounded reciprocal): q0 = fl(v * r) is within 1.5 ulps of the quotient; the
// first residual step (the residual v - sq * q0 is exact with a fused
// multiply-add) brings it within one ulp, and the second gives the correctly
// rounded quotient (Markstein's theorem for division by a reciprocal and
// residual corrections).  That holds while the residuals do not underflow and
// the quotient does not overflow: for 2^-126 <= |quotient| < 2^127.  Smaller
// quotients all have magnitude index 0 (only their sign matters, which the
// callers take from t0); callers clamp larger ones first.
__device__ __forceinline__ float exact_quotient(float v, float sq, float r)
{
    const float q0 = v * r;
    const float q1 = __builtin_fmaf(__builtin_fmaf(-q0, sq, v), r, q0);
    return __builtin_fmaf(__builtin_fmaf(-q1, sq, v), r, q1);
}

// ---------------------------------------------------------------- per-scale-byte table
//
// Everything a block needs beyond its own data depends only on its E4M3 scale
// byte S (0..0x7E), so each workgroup tabulates it once, for all 128 bytes, in
// LDS.  Entry for S (4 dwords, 16 bytes):
//   [0]  r ~ 1 / sq (binary32 bits), the multiplier of the fast path; the sign
//        bit is set when the fast path is NOT exact under this S
//   [1]  sd = decode(S) / gs (binary32 bits), the factor of the outputs
//   [2]  fl(1 / sq) (binary32 bits), the reciprocal of the exact-quotient path
//   [3]  t7 | (t0 - 1) << 16
// t_i (i = 1..7) is the smallest magnitude bit pattern whose E2M1 index is >= i;
// t0 the smallest whose quotient is nonzero.
//
// Fast path: q' = fl(x * r) goes through the gfx950 FP4 converter, which rounds
// a binary32 value to E2M1 with ties to even (checked on every binary32 input).
// q' can differ from the exact quotient fl(x / sq) in its last bits, and the
// code differs only if some bf16 magnitude lands on different sides of a
// decision boundary.  Both decisions are monotone in |x|, so comparing them at
// the two bf16 values around each exact threshold t_i settles it for every
// input.  Under an S that fails (or whose t0 is not 1), codes come from the
// correctly rounded quotient fl(x / sq) itself (exact_quotient), which is right
// under every S; a wave with any such block takes that path for all its lanes.
constexpr int kEntryWords = 4;
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
    dst[2] = r0;
    dst[3] = t7 | ((t0 - 1u) << 16);
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

// Codes of one bf16 pair into byte P of `out` from the correctly rounded
// quotients, under any scale byte: magnitudes are clamped at t7 (every larger
// one has index 7 too), so the quotient stays below about 5 and finite; the
// sign is kept only where |x| >= t0, so -0 and negative values whose quotient
// rounds to zero give code 0 (the method signs a code only when the quotient
// is below zero).  t7x2 and t0m1x2 hold the thresholds in both halves.
template <int P>
__device__ __forceinline__ uint32_t code_pair_exact(uint32_t out, uint32_t w, float sq, float r, uint32_t t7x2,
                                                    uint32_t t0m1x2)
{
    const uint32_t m = w & 0x7FFF7FFFu;
    const uint32_t v = pk_min(m, t7x2) | (w & pk_sub(t0m1x2, m) & 0x80008000u);
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, exact_quotient(__uint_as_float(v << 16), sq, r),
                                                    exact_quotient(__uint_as_float(v & 0xFFFF0000u), sq, r),
                                                    1.0f, P);
}

// Codes of four bf16 pairs as one dword of nibbles, exact-quotient path.
__device__ __forceinline__ uint32_t codes_exact(const uint32_t* w, const uint32_t* e)
{
    const float sd = __uint_as_float(e[1]);
    const float sq = sd < kEps ? kEps : sd;
    const float r = __uint_as_float(e[2]);
    const uint32_t t7x2 = (e[3] & 0xFFFFu) * 0x10001u;
    const uint32_t t0m1x2 = (e[3] >> 16) * 0x10001u;
    uint32_t out = 0;
    out = code_pair_exact<0>(out, w[0], sq, r, t7x2, t0m1x2);
    out = code_pair_exact<1>(out, w[1], sq, r, t7x2, t0m1x2);
    out = code_pair_exact<2>(out, w[2], sq, r, t7x2, t0m1x2);
    out = code_pair_exact<3>(out, w[3], sq, r, t7x2, t0m1x2);
    return out;
}

// The eight codes of four bf16 pairs (one dword of nibbles) under table entry e.
// One path per wave: the fast one when every lane's scale byte passed the check,
// else the exact quotient for all lanes (right under every scale byte).
__device__ __forceinline__ uint32_t half_codes(const uint32_t* w, const uint32_t* e)
{
    const uint32_t head = e[0];
    if (NVFP4_EXACT_PATH != 2 && __builtin_amdgcn_ballot_w64((head & kNotFast) != 0u) == 0u)
        return codes_fast(w, __uint_as_float(head));
    return codes_exact(w, e);
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

}  // namespace

#endif  // NVFP4_DEVICE_HPP
