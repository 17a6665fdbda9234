// The MXFP4 variant of libnvfp4 (included by nvfp4.hip): 32-element blocks with
// one binary32 scale each and no per-tensor factor (VideoX-Fun page, module
// constants: the block-size comment, which names 32-element blocks with a
// single-precision scale as the MXFP4 form).  Per block of
// one row:
//   s = block_amax / 6 (binary32);  q = x / max(s, 1e-12);
//   code = E2M1 round-to-nearest-even of min(|q|, 6), signed when q < 0;
//   fake-quant / unpack output = bf16_RNE(LUT[code] * s).
// A row whose length is not a multiple of 32 is zero-padded to whole blocks.

#ifndef NVFP4_MX_HPP
#define NVFP4_MX_HPP

#include "kernels.hpp"

namespace {

constexpr int64_t kMxBlock = 32;

// Quarter blocks: lanes 4k .. 4k+3 hold the four 8-element quarters of one block
// (16 bytes of bf16 each), so every load and store is contiguous across a wave,
// as with the NVFP4 half blocks.  Whole-block tensors have a multiple of four
// quarters, and every guard compares the four lanes of an aligned quad alike, so
// the lanes of a block are all active or all inactive at the permutes.

// Largest magnitude (bf16 bits) of the block whose quarter this lane holds: its
// own four dwords, then the quad's maximum by two DPP quad permutes
// ([1, 0, 3, 2], then [2, 3, 0, 1]).
__device__ __forceinline__ uint32_t quad_max(const uint32_t (&w)[4])
{
    const uint32_t mx = pk_max(pk_max(w[0] & 0x7FFF7FFFu, w[1] & 0x7FFF7FFFu),
                               pk_max(w[2] & 0x7FFF7FFFu, w[3] & 0x7FFF7FFFu));
    uint32_t m = max(mx & 0xFFFFu, mx >> 16);
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp((int)m, (int)m, 0xB1, 0xF, 0xF, false));
    return max(m, (uint32_t)__builtin_amdgcn_update_dpp((int)m, (int)m, 0x4E, 0xF, 0xF, false));
}

// The block scale bamax / 6 for a block maximum with bf16 bits bm: the binary64
// product with 1/6 rounded to binary32 is the correctly rounded quotient for
// every bf16 value (8 significant bits), as in scale_byte_of.
__device__ __forceinline__ float mx_scale_of(uint32_t bm)
{
    return (float)((double)bf16_value(bm) * (1.0 / 6.0));
}

// What a block's element codes need from its scale s: the divisor sq = max(s,
// 1e-12), its correctly rounded reciprocal r (one IEEE divide per block), and
// t0, the smallest bf16 magnitude whose quotient by sq rounds to a nonzero value
// (|x| / sq > 2^-150; sq * 2^-150 is exact in binary64), as (t0 - 1) in both
// halves of a dword.
struct MxDivisor {
    float sq, r;
    uint32_t t0m1;
};

__device__ __forceinline__ MxDivisor mx_divisor(float s)
{
    MxDivisor d;
    d.sq = s < kEps ? kEps : s;
    d.r = 1.0f / d.sq;
    d.t0m1 = (first_above((double)d.sq * 0x1p-150) - 1u) * 0x10001u;
    return d;
}

// fl(v / sq) by the reciprocal and two residual corrections (exact_quotient).
// |v| <= the block max, so the quotient is at most about 6 and never overflows;
// quotients below 2^-126 have magnitude index 0, and mx_code_pair takes their
// sign from t0.
__device__ __forceinline__ float mx_quotient(float v, const MxDivisor& d)
{
    return exact_quotient(v, d.sq, d.r);
}

// Codes of one bf16 pair into byte P of `out` through the FP4 converter (round to
// nearest even, saturating at 6, code sign from the input's sign bit).  The sign
// of an element is kept only where its quotient is nonzero (|x| >= t0), so -0
// and negative values whose quotient rounds to zero give code 0, as the method
// signs a code only when the quotient is below zero.
template <int P>
__device__ __forceinline__ uint32_t mx_code_pair(uint32_t out, uint32_t w, const MxDivisor& d)
{
    const uint32_t m = w & 0x7FFF7FFFu;
    const uint32_t v = m | (w & pk_sub(d.t0m1, m) & 0x80008000u);
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, mx_quotient(__uint_as_float(v << 16), d),
                                                    mx_quotient(__uint_as_float(v & 0xFFFF0000u), d), 1.0f, P);
}

// The eight codes of four bf16 pairs as one dword of nibbles.
__device__ __forceinline__ uint32_t mx_codes(const uint32_t* w, const MxDivisor& d)
{
    uint32_t out = 0;
    out = mx_code_pair<0>(out, w[0], d);
    out = mx_code_pair<1>(out, w[1], d);
    out = mx_code_pair<2>(out, w[2], d);
    out = mx_code_pair<3>(out, w[3], d);
    return out;
}

// One pass over the quarters with a grid stride: body(w, j) gets the four dwords
// of quarter j.  All of an iteration's loads are issued before its first body.
template <bool NtLd, typename Body>
__device__ __forceinline__ void mx_pass(const uint4* x, int64_t nquarters, Body body)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads * kUnroll;
    for (int64_t base = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; base < nquarters;
         base += stride) {
        uint4 v[kUnroll];
        load_halves<NtLd>(x, base, nquarters, v);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t j = walk(base + (int64_t)u * kThreads, nquarters);
            if (j >= 0) {
                const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
                body(w, j);
            }
        }
    }
}

__global__ __launch_bounds__(kThreads) void k_mx_fake_quant(const uint4* x, uint4* y, int64_t nquarters)
{
    mx_pass<NVFP4_FQ_NT_LD != 0>(x, nquarters, [&](const uint32_t (&w)[4], int64_t j) {
        const float s = mx_scale_of(quad_max(w));
        store16<NVFP4_FQ_NT_ST != 0>(y + j, decode_half(mx_codes(w, mx_divisor(s)), s));
    });
}

// Lane j stores the eight codes of quarter j (one dword of the packed codes); the
// first lane of a block also stores its scale.
__global__ __launch_bounds__(kThreads) void k_mx_quantize_pack(const uint4* __restrict__ x,
                                                               uint32_t* __restrict__ packed,
                                                               float* __restrict__ scales, int64_t nquarters)
{
    mx_pass<NVFP4_QP_NT_LD != 0>(x, nquarters, [&](const uint32_t (&w)[4], int64_t j) {
        const float s = mx_scale_of(quad_max(w));
        store4<NVFP4_QP_NT_ST != 0>(packed + j, mx_codes(w, mx_divisor(s)));
        if (!(j & 3))
            store4<NVFP4_MX_SC_NT != 0>(reinterpret_cast<uint32_t*>(scales) + (j >> 2), __float_as_uint(s));
    });
}

// Lane j decodes dword j of the packed codes (quarter j % 4 of block j / 4) with
// that block's scale and writes its eight bf16 outputs, 16 bytes at j.
__global__ __launch_bounds__(kThreads) void k_mx_dequant_unpack(const uint32_t* __restrict__ packed,
                                                                const float* __restrict__ scales,
                                                                uint4* __restrict__ y, int64_t nquarters)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads * kDqUnroll;
    for (int64_t base = (int64_t)blockIdx.x * kThreads * kDqUnroll + threadIdx.x; base < nquarters;
         base += stride) {
        uint32_t p[kDqUnroll];
        float s[kDqUnroll];
#pragma unroll
        for (int u = 0; u < kDqUnroll; ++u) {
            const int64_t j = base + (int64_t)u * kThreads;
            p[u] = j < nquarters ? packed[j] : 0u;
            s[u] = j < nquarters ? scales[j >> 2] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kDqUnroll; ++u) {
            const int64_t j = base + (int64_t)u * kThreads;
            if (j < nquarters)
                store16<NVFP4_DQ_NT_ST != 0>(y + j, decode_half(p[u], s[u]));
        }
    }
}

// ---------------------------------------------------------------- ragged rows, quarter-block lanes
//
// Rows whose length is not a multiple of 32, over the zero-padded rows, on the
// quarter-block lanes of the whole-block kernels: padded quarter j is the same
// 8-element unit of a row as a half block of the NVFP4 row kernels (HalfRows with
// 4 ceil(cols / 32) units per padded row), loaded and stored with dword accesses
// for even lengths and element by element for odd ones.  Quarter counts are
// multiples of 4, so the four lanes of a block are all active or all inactive at
// the quad max.
template <bool Odd, typename Body>
__device__ __forceinline__ void mx_rows_pass(const HalfRows& g, Body body)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads * kUnroll;
    for (int64_t base = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; base < g.nhalves; base += stride) {
        uint32_t w[kUnroll][4];
        int n[kUnroll];
        int64_t e[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t j = base + (int64_t)u * kThreads;
            n[u] = 0;
            e[u] = j < g.nhalves ? row_half(g, j, n[u]) : 0;
            load_row_half<Odd>(g.x, e[u], n[u], w[u]);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t j = base + (int64_t)u * kThreads;
            if (j < g.nhalves)
                body(w[u], j, e[u], n[u]);
        }
    }
}

template <bool Odd>
__global__ __launch_bounds__(kThreads) void k_mx_fake_quant_rows(HalfRows g, uint16_t* y)
{
    mx_rows_pass<Odd>(g, [&](const uint32_t (&w)[4], int64_t, int64_t e, int n) {
        const float s = mx_scale_of(quad_max(w));
        store_row_half<Odd>(y, e, n, decode_half(mx_codes(w, mx_divisor(s)), s));
    });
}

template <bool Odd>
__global__ __launch_bounds__(kThreads) void k_mx_quantize_pack_rows(HalfRows g, uint32_t* __restrict__ packed,
                                                                    float* __restrict__ scales)
{
    mx_rows_pass<Odd>(g, [&](const uint32_t (&w)[4], int64_t j, int64_t, int) {
        const float s = mx_scale_of(quad_max(w));
        store4<NVFP4_QP_NT_ST != 0>(packed + j, mx_codes(w, mx_divisor(s)));
        if (!(j & 3))
            store4<NVFP4_MX_SC_NT != 0>(reinterpret_cast<uint32_t*>(scales) + (j >> 2), __float_as_uint(s));
    });
}

template <bool Odd>
__global__ __launch_bounds__(kThreads) void k_mx_dequant_unpack_rows(const uint32_t* __restrict__ packed,
                                                                     const float* __restrict__ scales,
                                                                     uint16_t* __restrict__ y, HalfRows g)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads * kDqUnroll;
    for (int64_t base = (int64_t)blockIdx.x * kThreads * kDqUnroll + threadIdx.x; base < g.nhalves;
         base += stride) {
        uint32_t p[kDqUnroll];
        float s[kDqUnroll];
#pragma unroll
        for (int u = 0; u < kDqUnroll; ++u) {
            const int64_t j = base + (int64_t)u * kThreads;
            p[u] = j < g.nhalves ? packed[j] : 0u;
            s[u] = j < g.nhalves ? scales[j >> 2] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < kDqUnroll; ++u) {
            const int64_t j = base + (int64_t)u * kThreads;
            if (j < g.nhalves) {
                int n;
                const int64_t e = row_half(g, j, n);
                store_row_half<Odd>(y, e, n, decode_half(p[u], s[u]));
            }
        }
    }
}

// ---------------------------------------------------------------- ragged rows, one lane per block
//
// The same for tensors of 2^30 blocks and more: one lane per block, elements loaded
// and stored one at a time and masked at the row end (rows may start at any
// element).  Codes and scales keep the padded layout: block f is bytes 16f ..
// 16f + 15 of the packed codes and scale f.

// First element and element count of block f.
__device__ __forceinline__ int64_t mx_ragged_block(const RaggedShape& g, int64_t f, int& n)
{
    const int64_t r = f / g.nbr;
    const int64_t c0 = (f - r * g.nbr) * kMxBlock;
    const int64_t left = g.cols - c0;
    n = left < kMxBlock ? (int)left : (int)kMxBlock;
    return r * g.cols + c0;
}

// The 32 elements of block f (zeros past the row end) as 16 dwords, its scale and its codes.
__device__ __forceinline__ void mx_ragged_codes(const uint16_t* x, int64_t e0, int n, float& s, uint4& codes)
{
    uint32_t w[16];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        uint32_t (&half)[8] = *reinterpret_cast<uint32_t(*)[8]>(w + 8 * h);
        load_ragged(x, e0 + 16 * h, n - 16 * h, half);
    }
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i)
        mx = pk_max(mx, w[i] & 0x7FFF7FFFu);
    s = mx_scale_of(max(mx & 0xFFFFu, mx >> 16));
    const MxDivisor d = mx_divisor(s);
    codes = make_uint4(mx_codes(w, d), mx_codes(w + 4, d), mx_codes(w + 8, d), mx_codes(w + 12, d));
}

__global__ __launch_bounds__(kThreads) void k_mx_fake_quant_ragged(const uint16_t* x, uint16_t* y, RaggedShape g)
{
    for (int64_t f = (int64_t)blockIdx.x * kThreads + threadIdx.x; f < g.nblocks;
         f += (int64_t)gridDim.x * kThreads) {
        int n;
        const int64_t e0 = mx_ragged_block(g, f, n);
        float s;
        uint4 c;
        mx_ragged_codes(x, e0, n, s, c);
        store_ragged(y, e0, n, c.x, c.y, s);
        store_ragged(y, e0 + 16, n - 16, c.z, c.w, s);
    }
}

__global__ __launch_bounds__(kThreads) void k_mx_quantize_pack_ragged(const uint16_t* __restrict__ x,
                                                                      uint4* __restrict__ packed,
                                                                      float* __restrict__ scales, RaggedShape g)
{
    for (int64_t f = (int64_t)blockIdx.x * kThreads + threadIdx.x; f < g.nblocks;
         f += (int64_t)gridDim.x * kThreads) {
        int n;
        const int64_t e0 = mx_ragged_block(g, f, n);
        float s;
        uint4 c;
        mx_ragged_codes(x, e0, n, s, c);
        packed[f] = c;
        scales[f] = s;
    }
}

__global__ __launch_bounds__(kThreads) void k_mx_dequant_unpack_ragged(const uint4* __restrict__ packed,
                                                                       const float* __restrict__ scales,
                                                                       uint16_t* __restrict__ y, RaggedShape g)
{
    for (int64_t f = (int64_t)blockIdx.x * kThreads + threadIdx.x; f < g.nblocks;
         f += (int64_t)gridDim.x * kThreads) {
        int n;
        const int64_t e0 = mx_ragged_block(g, f, n);
        const uint4 c = packed[f];
        const float s = scales[f];
        store_ragged(y, e0, n, c.x, c.y, s);
        store_ragged(y, e0 + 16, n - 16, c.z, c.w, s);
    }
}

}  // namespace

#endif  // NVFP4_MX_HPP
