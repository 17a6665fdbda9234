/*
 * Host driver for the oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
 * (test infrastructure: tests/test_oracle_sanitize.py builds and runs it).
 *
 * Every buffer is malloc'ed at exactly the size the oracle's contract gives it, so a
 * read or write one byte past a row, a block, a pad or a tensor is reported.  The
 * outputs are written to a file so the test can compare the sanitized build with the
 * oracle's normal build, byte for byte.
 *
 * Input file: a sequence of cases, each int64 rows, int64 cols, then rows*cols bf16
 * bit patterns; then int64 nf and nf float32 values for the element-wise forms.
 * Output file, per case: float amax, float gs, packed [rows, 8*nbr], scales [rows, nbr],
 * dequantized bf16 [rows, cols], fake-quant bf16 [rows, cols], and the MXFP4 variant's
 * packed [rows, 16*mbr], float scales [rows, mbr], dequantized and fake-quant bf16
 * (mbr = ceil(cols / 32)); then the group amax of all
 * cases; then for the nf floats: E4M3 codes, E2M1 codes of |v|, bf16 roundings; then
 * the 256 E4M3 decodes; then the observer on each of the first min(nf, 64) floats.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

float nvo_amax(const uint16_t* x, int64_t n);
float nvo_amax_group(const uint16_t* const* xs, const int64_t* ns, int count);
float nvo_observer(float state, float cur, int mode, float decay);
float nvo_global_scale(float amax);
void nvo_quantize(const uint16_t* x, int64_t rows, int64_t cols, float amax,
                  uint8_t* packed, uint8_t* scales, float* gs_out);
void nvo_dequantize(const uint8_t* packed, const uint8_t* scales, float gs,
                    int64_t rows, int64_t cols, uint16_t* y);
int nvo_fake_quant(const uint16_t* x, uint16_t* y, int64_t rows, int64_t cols, float amax);
void nvo_e4m3_encode_array(const float* v, uint8_t* out, int64_t n);
void nvo_e4m3_decode_array(const uint8_t* b, float* out, int64_t n);
void nvo_e2m1_round_array(const float* a, uint8_t* out, int64_t n);
void nvo_f32_to_bf16_array(const float* f, uint16_t* out, int64_t n);
void nvo_mx_quantize(const uint16_t* x, int64_t rows, int64_t cols, uint8_t* packed, float* scales);
void nvo_mx_dequantize(const uint8_t* packed, const float* scales, int64_t rows, int64_t cols, uint16_t* y);
int nvo_mx_fake_quant(const uint16_t* x, uint16_t* y, int64_t rows, int64_t cols);

#define MAX_CASES 64

static void* exact(size_t n)
{
    /* malloc(0) may return NULL; the oracle never dereferences an empty buffer, so a
     * one-byte allocation stands in and any access to it is still out of bounds */
    void* p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "allocation of %zu bytes failed\n", n);
        exit(2);
    }
    return p;
}

static void put(FILE* f, const void* p, size_t n)
{
    if (n && fwrite(p, 1, n, f) != n) {
        fprintf(stderr, "short write\n");
        exit(2);
    }
}

int main(int argc, char** argv)
{
    if (argc != 3) {
        fprintf(stderr, "usage: %s input output\n", argv[0]);
        return 2;
    }
    FILE* in = fopen(argv[1], "rb");
    FILE* out = fopen(argv[2], "wb");
    if (!in || !out) {
        fprintf(stderr, "cannot open files\n");
        return 2;
    }
    int64_t ncases;
    if (fread(&ncases, 8, 1, in) != 1 || ncases < 0 || ncases > MAX_CASES)
        return 2;
    uint16_t* xs[MAX_CASES];
    int64_t ns[MAX_CASES];
    for (int64_t c = 0; c < ncases; c++) {
        int64_t rc[2];
        if (fread(rc, 8, 2, in) != 2 || rc[0] < 0 || rc[1] < 1)
            return 2;
        int64_t rows = rc[0], cols = rc[1], n = rows * cols;
        int64_t nbr = (cols + 15) / 16;
        uint16_t* x = (uint16_t*)exact((size_t)n * 2);
        if (n && fread(x, 2, (size_t)n, in) != (size_t)n)
            return 2;
        uint8_t* packed = (uint8_t*)exact((size_t)(rows * 8 * nbr));
        uint8_t* scales = (uint8_t*)exact((size_t)(rows * nbr));
        uint16_t* dq = (uint16_t*)exact((size_t)n * 2);
        uint16_t* fq = (uint16_t*)exact((size_t)n * 2);
        float amax = nvo_amax(x, n), gs;
        nvo_quantize(x, rows, cols, amax, packed, scales, &gs);
        nvo_dequantize(packed, scales, gs, rows, cols, dq);
        if (nvo_fake_quant(x, fq, rows, cols, amax) != 0)
            return 3;
        put(out, &amax, 4);
        put(out, &gs, 4);
        put(out, packed, (size_t)(rows * 8 * nbr));
        put(out, scales, (size_t)(rows * nbr));
        put(out, dq, (size_t)n * 2);
        put(out, fq, (size_t)n * 2);
        int64_t mbr = (cols + 31) / 32;
        uint8_t* mpacked = (uint8_t*)exact((size_t)(rows * 16 * mbr));
        float* mscales = (float*)exact((size_t)(rows * mbr) * 4);
        nvo_mx_quantize(x, rows, cols, mpacked, mscales);
        nvo_mx_dequantize(mpacked, mscales, rows, cols, dq);
        if (nvo_mx_fake_quant(x, fq, rows, cols) != 0)
            return 3;
        put(out, mpacked, (size_t)(rows * 16 * mbr));
        put(out, mscales, (size_t)(rows * mbr) * 4);
        put(out, dq, (size_t)n * 2);
        put(out, fq, (size_t)n * 2);
        free(mpacked);
        free(mscales);
        free(packed);
        free(scales);
        free(dq);
        free(fq);
        xs[c] = x;
        ns[c] = n;
    }
    float g = nvo_amax_group((const uint16_t* const*)xs, ns, (int)ncases);
    put(out, &g, 4);
    for (int64_t c = 0; c < ncases; c++)
        free(xs[c]);

    int64_t nf;
    if (fread(&nf, 8, 1, in) != 1 || nf < 0 || nf > (1 << 24))
        return 2;
    float* v = (float*)exact((size_t)nf * 4);
    float* mag = (float*)exact((size_t)nf * 4);
    if (nf && fread(v, 4, (size_t)nf, in) != (size_t)nf)
        return 2;
    for (int64_t i = 0; i < nf; i++)
        mag[i] = fabsf(v[i]);
    uint8_t* e4 = (uint8_t*)exact((size_t)nf);
    uint8_t* e2 = (uint8_t*)exact((size_t)nf);
    uint16_t* b16 = (uint16_t*)exact((size_t)nf * 2);
    nvo_e4m3_encode_array(v, e4, nf);
    nvo_e2m1_round_array(mag, e2, nf);
    nvo_f32_to_bf16_array(v, b16, nf);
    put(out, e4, (size_t)nf);
    put(out, e2, (size_t)nf);
    put(out, b16, (size_t)nf * 2);
    uint8_t bytes[256];
    float dec[256];
    for (int i = 0; i < 256; i++)
        bytes[i] = (uint8_t)i;
    nvo_e4m3_decode_array(bytes, dec, 256);
    put(out, dec, sizeof dec);
    for (int64_t i = 0; i < nf && i < 64; i++) {
        float s0 = nvo_observer(-1.0f, mag[i], 0, 0.0f);
        float s1 = nvo_observer(mag[i], 2.0f * mag[i] + 1.0f, 0, 0.0f);
        float s2 = nvo_observer(mag[i], 0.5f, 1, 0.01f);
        float s3 = nvo_global_scale(mag[i]);
        put(out, &s0, 4);
        put(out, &s1, 4);
        put(out, &s2, 4);
        put(out, &s3, 4);
    }
    free(v);
    free(mag);
    free(e4);
    free(e2);
    free(b16);
    fclose(in);
    if (fclose(out) != 0)
        return 2;
    return 0;
}
