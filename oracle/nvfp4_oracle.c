/*
 * NVFP4 two-level block quantization -- CPU ORACLE (test infrastructure only).
 *
 * This file is the plain, slow, scalar statement of what the quantizer computes.
 * It exists to check the HIP library against; it is not part of the product
 * path.  Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark load it.  It shares no code, header, table or helper with the HIP
 * library.
 *
 * Build: any C99 compiler, -O2 -ffp-contract=off, no fast-math, no FTZ/DAZ.
 * On x86-64 float arithmetic is SSE binary32: every +,-,*,/ below is one IEEE
 * round-to-nearest-even operation, and subnormals are kept.
 *
 * Sources (the pages):
 *   [VX]  VideoX-Fun page "videox_fun/utils/fp4_optimization.py" (gpu_memory_mode
 *         branch): the module constants, _float4_round, quantize_weight_to_float4,
 *         dequantize_weight_from_float4.  Authority for every numeric detail.
 *   [QAT] verl tutorial page "linear.py -- QATLinear" (verl.utils.qat.linear):
 *         section 1 (Triton FP4 fake-quant kernel), 2 (straight-through
 *         estimator), 4 (weight fake-quant with fused siblings), 5 (activation
 *         observer strategy).
 *   [FT]  "FasterTransformer quantization deep dive" page, FP8 format table
 *         (E4M3 range +-448).
 *   [KS]  "Kuaishou AI Infra internship" interview-notes page, question on FP4
 *         data distribution (E2M1 positive values 0 .. 6).
 *
 * Readings where the pages are silent or disagree (each also stated at its use):
 *   R1  all divisions are IEEE binary32 divisions (the torch listing's
 *       scalar/tensor form is evaluated differently by torch; the exact reading
 *       is the plain quotient);
 *   R2  the E4M3 cast rounds to nearest-even and saturates at 448 (torch's cast
 *       turns values above 464 into NaN instead);
 *   R3  the per-tensor factor divides ([VX]), it does not multiply ([QAT] s.1);
 *   R4  fake-quant is quantize followed by dequantize, so the fake-quant output
 *       multiplies by the unclamped decoded block scale;
 *   R5  the observer state -1 means "no observation yet": the first update
 *       stores the current amax for both observer kinds;
 *   R6  a row whose length is not a multiple of 16 is zero-padded to the next
 *       multiple ([VX] quantize_weight_to_float4), and the unpack drops the pad;
 *   R7  the MXFP4 variant ([VX] module constants, the block-size comment: 32-element
 *       blocks with a single-precision scale)
 *       is NVFP4's block step with 32-element blocks, the block scale kept in
 *       binary32 as block_amax / 6 (no per-tensor factor, no E4M3 rounding),
 *       the same clamp before it divides the elements, and the same element
 *       rounding, sign rule and output product.
 *
 * Parity pins (tests/test_oracle_pins.py): E2M1 grid and ties against the
 * pages' printed values and a brute-force nearest-value search; E4M3 encode and
 * decode against torch's float8_e4m3fn CPU cast; bf16 rounding against torch's
 * bfloat16 CPU cast; the all-codes x all-scales tensor; exact tie tensors;
 * pack/unpack identities; observer closed forms; special cases.  No page prints
 * a worked quantization example, so whole-tensor outputs on random inputs are
 * pinned only through these pieces and an independent numpy/torch
 * re-derivation on small tensors.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- constants ([VX] module constants; [FT] FP8 table; [KS]) ---------------- */
#define E2M1_MAX 6.0f         /* largest E2M1 magnitude                            */
#define BLOCK 16              /* NVFP4 block width                                  */
#define E4M3_MAX 448.0f       /* largest finite float8_e4m3fn                       */
#define SCALE_EPS 1e-12f      /* the clamp(min=1e-12) applied in binary32           */

/* E2M1 magnitudes; index = code & 7 ([VX] FLOAT4_MAGNITUDES, [KS]).                */
static const float MAGNITUDE[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

static float f32_of_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_of_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* ---- bf16 ------------------------------------------------------------------- */

/* bf16 -> binary32 is exact: the bf16 pattern is the upper half of the float.    */
float nvo_bf16_to_f32(uint16_t h) { return f32_of_bits((uint32_t)h << 16); }

/* binary32 -> bf16, round to nearest, ties to even, by the definition: keep the
 * upper 16 bits and add one unit when the dropped half is above one half unit,
 * or exactly one half unit while the kept part is odd.  NaN stays a quiet NaN.  */
uint16_t nvo_f32_to_bf16(float f)
{
    uint32_t u = bits_of_f32(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t kept = u >> 16, dropped = u & 0xFFFFu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))
        kept += 1u;   /* a carry into the exponent is the correct next value */
    return (uint16_t)kept;
}

/* ---- E4M3 (float8_e4m3fn) ----------------------------------------------------
 * Format: sign bit 7, exponent bits 6..3 with bias 7, mantissa bits 2..0.
 * Exponent field 0 holds the subnormals m * 2^-9.  0x7F / 0xFF are NaN; there is
 * no infinity, so the largest finite value is 0x7E = 1.75 * 2^8 = 448.           */
float nvo_e4m3_decode(uint8_t b)
{
    int sign = b >> 7, e = (b >> 3) & 0xF, m = b & 7;
    float mag;
    if (e == 0xF && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexpf((float)m, -9);
    else
        mag = ldexpf(1.0f + (float)m / 8.0f, e - 7);
    return sign ? -mag : mag;
}

/* Non-negative binary32 -> E4M3 byte, round to nearest with ties to the even
 * byte, saturating at 448 (reading R2).  Codes 0x00..0x7E decode to increasing
 * values, so a bisection over them finds the two neighbours of v; their
 * mid-point has at most five significant bits and is exact in double.           */
uint8_t nvo_e4m3_encode(float v)
{
    if (!(v < E4M3_MAX))                 /* v >= 448 saturates (NaN too)           */
        return 0x7E;
    if (v <= 0.0f)
        return 0x00;
    int lo = 0, hi = 0x7E;               /* decode(lo) <= v < decode(hi)            */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (nvo_e4m3_decode((uint8_t)mid) <= v)
            lo = mid;
        else
            hi = mid;
    }
    double below = nvo_e4m3_decode((uint8_t)lo);
    double above = nvo_e4m3_decode((uint8_t)(lo + 1));
    double mid = (below + above) / 2.0;
    if ((double)v < mid) return (uint8_t)lo;
    if ((double)v > mid) return (uint8_t)(lo + 1);
    return (uint8_t)((lo % 2 == 0) ? lo : lo + 1);
}

/* ---- E2M1 rounding ([VX] _float4_round) --------------------------------------
 * A non-negative value goes to the nearest of the eight magnitudes.  When it sits
 * exactly half-way between two neighbours, the one with the even index wins (the
 * even E2M1 mantissa bit).  Anything at or above the largest magnitude maps to it.
 * The two neighbours are found by a walk up the sorted magnitudes; their
 * mid-point has at most four significant bits, so it is exact in double.         */
int nvo_e2m1_round(float a)
{
    if (!(a < MAGNITUDE[7]))
        return 7;
    int lo = 0;                          /* MAGNITUDE[lo] <= a < MAGNITUDE[lo + 1]  */
    while (lo < 6 && MAGNITUDE[lo + 1] <= a)
        lo++;
    double mid = ((double)MAGNITUDE[lo] + (double)MAGNITUDE[lo + 1]) / 2.0;
    if ((double)a < mid) return lo;
    if ((double)a > mid) return lo + 1;
    return (lo % 2 == 0) ? lo : lo + 1;
}

/* ---- step 1: per-tensor amax ([VX] quantize_weight_to_float4; [QAT] s.4) ----- */
float nvo_amax(const uint16_t* x, int64_t n)
{
    float m = 0.0f;
    for (int64_t i = 0; i < n; i++) {
        float a = fabsf(nvo_bf16_to_f32(x[i]));
        if (a > m)
            m = a;
    }
    return m;
}

/* Shared amax of fused siblings: the max over every sibling's amax ([QAT] s.4).  */
float nvo_amax_group(const uint16_t* const* xs, const int64_t* ns, int count)
{
    float m = 0.0f;
    for (int k = 0; k < count; k++) {
        float a = nvo_amax(xs[k], ns[k]);
        if (a > m)
            m = a;
    }
    return m;
}

/* ---- activation observer ([QAT] s.5) -------------------------------------------
 * mode 0 "static_minmax": the running maximum of the observed amax.
 * mode 1 exponential moving average with weight `decay` on the new observation
 * (the page names it "minmax"): (1 - d) * old + d * cur, each product and the
 * sum rounded separately.  Reading R5 for the -1 initial state.                  */
float nvo_observer(float state, float cur, int mode, float decay)
{
    if (state < 0.0f)
        return cur;
    if (mode == 0)
        return cur > state ? cur : state;
    float keep = 1.0f - decay;
    float a = keep * state;
    float b = decay * cur;
    return a + b;
}

/* ---- step 2: per-tensor factor ([VX] quantize_weight_to_float4) -------------
 * (E4M3_MAX * E2M1_MAX) / max(amax, 1e-12); 448 * 6 = 2688 is exact.            */
float nvo_global_scale(float amax)
{
    float clamped = amax < SCALE_EPS ? SCALE_EPS : amax;
    return (E4M3_MAX * E2M1_MAX) / clamped;
}

/* ---- steps 3 and 4: quantize and pack ([VX] quantize_weight_to_float4) ------
 * x: bf16 [rows, cols] row-major.  Rows are zero-padded to `padded` columns, a
 * multiple of 16 (reading R6).  Outputs: packed [rows, padded/2] bytes, the
 * even column in the low nibble; scales [rows, padded/16] E4M3 bytes; *gs_out
 * the per-tensor factor.  `amax` is the per-tensor (or shared, or observed)
 * amax the caller supplies.                                                      */
void nvo_quantize(const uint16_t* x, int64_t rows, int64_t cols, float amax,
                  uint8_t* packed, uint8_t* scales, float* gs_out)
{
    int64_t padded = (cols + BLOCK - 1) / BLOCK * BLOCK;
    int64_t nblk = padded / BLOCK;
    float gs = nvo_global_scale(amax);
    *gs_out = gs;
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t j = 0; j < nblk; j++) {
            float val[BLOCK];
            for (int i = 0; i < BLOCK; i++) {
                int64_t c = j * BLOCK + i;
                val[i] = c < cols ? nvo_bf16_to_f32(x[r * cols + c]) : 0.0f;
            }
            /* first-level scale: E4M3 of (block_amax / 6) * gs, read back and
             * divided by gs, clamped to 1e-12 before it divides the elements  */
            float block_amax = 0.0f;
            for (int i = 0; i < BLOCK; i++)
                if (fabsf(val[i]) > block_amax)
                    block_amax = fabsf(val[i]);
            uint8_t s8 = nvo_e4m3_encode((block_amax / E2M1_MAX) * gs);
            float block_scale = nvo_e4m3_decode(s8) / gs;
            if (block_scale < SCALE_EPS)
                block_scale = SCALE_EPS;
            scales[r * nblk + j] = s8;
            uint8_t code[BLOCK];
            for (int i = 0; i < BLOCK; i++) {
                float scaled = val[i] / block_scale;
                if (scaled > E2M1_MAX) scaled = E2M1_MAX;
                if (scaled < -E2M1_MAX) scaled = -E2M1_MAX;
                int idx = nvo_e2m1_round(fabsf(scaled));
                code[i] = (uint8_t)(scaled < 0.0f ? idx + 8 : idx);
            }
            for (int i = 0; i < BLOCK / 2; i++)
                packed[r * (padded / 2) + j * (BLOCK / 2) + i] =
                    (uint8_t)(code[2 * i] | (code[2 * i + 1] << 4));
        }
    }
}

/* ---- unpack ([VX] dequantize_weight_from_float4) -----------------------------
 * value = LUT[code] * (decode(scale) / gs), rounded to bf16; LUT[8..15] are the
 * negated magnitudes, so code 8 is -0.  Writes y [rows, cols].                   */
void nvo_dequantize(const uint8_t* packed, const uint8_t* scales, float gs,
                    int64_t rows, int64_t cols, uint16_t* y)
{
    int64_t padded = (cols + BLOCK - 1) / BLOCK * BLOCK;
    int64_t nblk = padded / BLOCK;
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t c = 0; c < cols; c++) {
            uint8_t byte = packed[r * (padded / 2) + c / 2];
            int code = (c % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
            float lut = (code & 8) ? -MAGNITUDE[code & 7] : MAGNITUDE[code & 7];
            float block_scale = nvo_e4m3_decode(scales[r * nblk + c / BLOCK]) / gs;
            y[r * cols + c] = nvo_f32_to_bf16(lut * block_scale);
        }
    }
}

/* ---- fake-quant (reading R4): quantize, then dequantize ----------------------
 * [QAT] s.1 emits the rescaled grid value in the input dtype; the QAT notes
 * ([KS]) describe fake quantization as quantize followed by dequantize.
 * The straight-through backward ([QAT] s.2) is the identity and needs no code.   */
int nvo_fake_quant(const uint16_t* x, uint16_t* y, int64_t rows, int64_t cols, float amax)
{
    int64_t padded = (cols + BLOCK - 1) / BLOCK * BLOCK;
    size_t np = (size_t)(rows * (padded / 2)), ns = (size_t)(rows * (padded / BLOCK));
    uint8_t* packed = (uint8_t*)malloc(np ? np : 1);
    uint8_t* scales = (uint8_t*)malloc(ns ? ns : 1);
    if (!packed || !scales) {
        free(packed);
        free(scales);
        return -1;
    }
    float gs;
    nvo_quantize(x, rows, cols, amax, packed, scales, &gs);
    nvo_dequantize(packed, scales, gs, rows, cols, y);
    free(packed);
    free(scales);
    return 0;
}

/* ---- MXFP4 variant (reading R7; [VX] module constants) ------------------------
 * Blocks of 32 consecutive elements of one row, a row zero-padded to a multiple
 * of 32.  Each block keeps one binary32 scale s = block_amax / 6 (a zero block
 * has s = 0); elements are divided by max(s, 1e-12), rounded onto the E2M1 grid
 * and signed exactly as in nvo_quantize; the unpack multiplies the signed
 * magnitude by s and rounds to bf16.  Outputs: packed [rows, padded / 2] bytes
 * (even column in the low nibble), scales [rows, padded / 32] binary32.          */
#define MX_BLOCK 32

void nvo_mx_quantize(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* packed, float* scales)
{
    int64_t padded = (cols + MX_BLOCK - 1) / MX_BLOCK * MX_BLOCK;
    int64_t nblk = padded / MX_BLOCK;
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t j = 0; j < nblk; j++) {
            float val[MX_BLOCK];
            for (int i = 0; i < MX_BLOCK; i++) {
                int64_t c = j * MX_BLOCK + i;
                val[i] = c < cols ? nvo_bf16_to_f32(x[r * cols + c]) : 0.0f;
            }
            float block_amax = 0.0f;
            for (int i = 0; i < MX_BLOCK; i++)
                if (fabsf(val[i]) > block_amax)
                    block_amax = fabsf(val[i]);
            float scale = block_amax / E2M1_MAX;
            scales[r * nblk + j] = scale;
            float divisor = scale < SCALE_EPS ? SCALE_EPS : scale;
            uint8_t code[MX_BLOCK];
            for (int i = 0; i < MX_BLOCK; i++) {
                float scaled = val[i] / divisor;
                if (scaled > E2M1_MAX) scaled = E2M1_MAX;
                if (scaled < -E2M1_MAX) scaled = -E2M1_MAX;
                int idx = nvo_e2m1_round(fabsf(scaled));
                code[i] = (uint8_t)(scaled < 0.0f ? idx + 8 : idx);
            }
            for (int i = 0; i < MX_BLOCK / 2; i++)
                packed[r * (padded / 2) + j * (MX_BLOCK / 2) + i] =
                    (uint8_t)(code[2 * i] | (code[2 * i + 1] << 4));
        }
    }
}

void nvo_mx_dequantize(const uint8_t* packed, const float* scales, int64_t rows, int64_t cols, uint16_t* y)
{
    int64_t padded = (cols + MX_BLOCK - 1) / MX_BLOCK * MX_BLOCK;
    int64_t nblk = padded / MX_BLOCK;
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t c = 0; c < cols; c++) {
            uint8_t byte = packed[r * (padded / 2) + c / 2];
            int code = (c % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
            float lut = (code & 8) ? -MAGNITUDE[code & 7] : MAGNITUDE[code & 7];
            y[r * cols + c] = nvo_f32_to_bf16(lut * scales[r * nblk + c / MX_BLOCK]);
        }
    }
}

/* MXFP4 fake-quant: quantize, then dequantize (as nvo_fake_quant). */
int nvo_mx_fake_quant(const uint16_t* x, uint16_t* y, int64_t rows, int64_t cols)
{
    int64_t padded = (cols + MX_BLOCK - 1) / MX_BLOCK * MX_BLOCK;
    size_t np = (size_t)(rows * (padded / 2)), ns = (size_t)(rows * (padded / MX_BLOCK));
    uint8_t* packed = (uint8_t*)malloc(np ? np : 1);
    float* scales = (float*)malloc((ns ? ns : 1) * sizeof(float));
    if (!packed || !scales) {
        free(packed);
        free(scales);
        return -1;
    }
    nvo_mx_quantize(x, rows, cols, packed, scales);
    nvo_mx_dequantize(packed, scales, rows, cols, y);
    free(packed);
    free(scales);
    return 0;
}

/* ---- element-wise array forms, for the pin tests ---------------------------- */
void nvo_e4m3_encode_array(const float* v, uint8_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = nvo_e4m3_encode(v[i]);
}

void nvo_e4m3_decode_array(const uint8_t* b, float* out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = nvo_e4m3_decode(b[i]);
}

void nvo_e2m1_round_array(const float* a, uint8_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = (uint8_t)nvo_e2m1_round(a[i]);
}

void nvo_f32_to_bf16_array(const float* f, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = nvo_f32_to_bf16(f[i]);
}
