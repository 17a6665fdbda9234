/*
 * The C ABI used from plain C, with no Python and no torch: HIP runtime calls
 * for memory and a stream, libnvfp4 for the work, and the CPU oracle (linked
 * in, test infrastructure) for the expected bytes.
 * tests/test_gpu_c_abi.py builds and runs it on a GPU.
 *
 * One seeded bf16 tensor (rows x cols, cols a multiple of 16 or not, given on
 * the command line) goes through the fused fake-quant (plain and workspace),
 * the fused quantize-pack, the dequant-unpack and the one-call observe step;
 * every device result must equal the oracle's bit for bit.
 * Exit status 0 and "all bit-exact" on success.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "nvfp4.h"

float nvo_amax(const uint16_t* x, int64_t n);
float nvo_observer(float state, float cur, int mode, float decay);
void nvo_quantize(const uint16_t* x, int64_t rows, int64_t cols, float amax,
                  uint8_t* packed, uint8_t* scales, float* gs_out);
void nvo_dequantize(const uint8_t* packed, const uint8_t* scales, float gs,
                    int64_t rows, int64_t cols, uint16_t* y);
int nvo_fake_quant(const uint16_t* x, uint16_t* y, int64_t rows, int64_t cols, float amax);

#define HIP_OK(call)                                                              \
    do {                                                                          \
        hipError_t e_ = (call);                                                   \
        if (e_ != hipSuccess) {                                                   \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));     \
            exit(2);                                                              \
        }                                                                         \
    } while (0)

#define NV_OK(call)                                                               \
    do {                                                                          \
        int s_ = (call);                                                          \
        if (s_ != NVFP4_OK) {                                                     \
            fprintf(stderr, "%s failed: %s\n", #call, nvfp4_strerror(s_));        \
            exit(3);                                                              \
        }                                                                         \
    } while (0)

static int failures = 0;

static void same(const void* got, const void* want, size_t bytes, const char* what)
{
    if (memcmp(got, want, bytes) != 0) {
        size_t i = 0;
        while (((const uint8_t*)got)[i] == ((const uint8_t*)want)[i])
            i++;
        fprintf(stderr, "%s: first differing byte %zu of %zu\n", what, i, bytes);
        failures++;
    }
}

static uint32_t bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

/* splitmix64: a seeded source of bf16 test values (normal-ish, wide exponent range). */
static uint64_t state_;
static uint64_t next64(void)
{
    uint64_t z = (state_ += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static void* device(size_t bytes)
{
    void* p = NULL;
    HIP_OK(hipMalloc(&p, bytes ? bytes : 1));
    return p;
}

int main(int argc, char** argv)
{
    if (argc != 4) {
        fprintf(stderr, "usage: %s rows cols seed\n", argv[0]);
        return 2;
    }
    const int64_t rows = atoll(argv[1]), cols = atoll(argv[2]);
    state_ = (uint64_t)atoll(argv[3]);
    const int64_t n = rows * cols, nbr = (cols + 15) / 16;
    const size_t xb = (size_t)n * 2, pb = (size_t)(rows * 8 * nbr), sb = (size_t)(rows * nbr);

    uint16_t* x = malloc(xb ? xb : 1);
    for (int64_t i = 0; i < n; i++) {
        /* sign, an exponent from a 12-binade window around 1, 7 random fraction bits */
        uint64_t r = next64();
        uint16_t e = (uint16_t)(127 - 6 + (r % 12));
        x[i] = (uint16_t)(((r >> 8) & 1) << 15 | e << 7 | ((r >> 16) & 0x7F));
        if ((r >> 40) % 97 == 0)
            x[i] = (uint16_t)((r >> 8) & 1) << 15;  /* some zeros and -0 */
    }

    /* the oracle */
    const float a = nvo_amax(x, n);
    uint16_t* fq_ref = malloc(xb ? xb : 1);
    uint8_t* p_ref = malloc(pb ? pb : 1);
    uint8_t* s_ref = malloc(sb ? sb : 1);
    uint16_t* dq_ref = malloc(xb ? xb : 1);
    float g_ref;
    if (nvo_fake_quant(x, fq_ref, rows, cols, a) != 0)
        return 2;
    nvo_quantize(x, rows, cols, a, p_ref, s_ref, &g_ref);
    nvo_dequantize(p_ref, s_ref, g_ref, rows, cols, dq_ref);
    const float prior = 0.5f * a, decay = 0.25f;
    const float st0_ref = nvo_observer(prior, a, NVFP4_OBS_STATIC_MINMAX, 0.0f);
    const float st1_ref = nvo_observer(prior, a, NVFP4_OBS_EMA, decay);
    uint16_t* ob0_ref = malloc(xb ? xb : 1);
    uint16_t* ob1_ref = malloc(xb ? xb : 1);
    if (nvo_fake_quant(x, ob0_ref, rows, cols, st0_ref) != 0 || nvo_fake_quant(x, ob1_ref, rows, cols, st1_ref) != 0)
        return 2;

    /* the device */
    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));
    void* dx = device(xb);
    void* dy = device(xb);
    void* dy1 = device(xb);
    uint8_t* dp = device(pb);
    uint8_t* ds = device(sb);
    float* scal = device(8 * sizeof(float));   /* amax, amax_ws, gs, cur, state0, state1 */
    void* ws = device(NVFP4_WORKSPACE_BYTES);
    HIP_OK(hipMemcpy(dx, x, xb, hipMemcpyHostToDevice));
    const float states[2] = {prior, prior};
    HIP_OK(hipMemcpy(scal + 4, states, sizeof states, hipMemcpyHostToDevice));

    uint16_t* got = malloc(xb ? xb : 1);
    uint8_t* gotp = malloc(pb ? pb : 1);
    uint8_t* gots = malloc(sb ? sb : 1);
    float sc[8];

    NV_OK(nvfp4_fake_quant(dx, dy, rows, cols, NULL, scal + 0, s));
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(got, dy, xb, hipMemcpyDeviceToHost));
    same(got, fq_ref, xb, "nvfp4_fake_quant");

    NV_OK(nvfp4_fake_quant_ws(dx, dy, rows, cols, scal + 1, ws, s));
    NV_OK(nvfp4_quantize_pack(dx, rows, cols, NULL, scal + 0, dp, ds, scal + 2, s));
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(got, dy, xb, hipMemcpyDeviceToHost));
    same(got, fq_ref, xb, "nvfp4_fake_quant_ws");
    HIP_OK(hipMemcpy(gotp, dp, pb, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(gots, ds, sb, hipMemcpyDeviceToHost));
    same(gotp, p_ref, pb, "nvfp4_quantize_pack codes");
    same(gots, s_ref, sb, "nvfp4_quantize_pack scales");

    NV_OK(nvfp4_dequant_unpack(dp, ds, scal + 2, rows, cols, dy, s));
    NV_OK(nvfp4_observe_fake_quant(dx, rows, cols, scal + 3, scal + 4, NVFP4_OBS_STATIC_MINMAX, 0.0f, dy1,
                                   scal + 5, NVFP4_OBS_EMA, decay, dx, ws, s));   /* y1 in place */
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(got, dy, xb, hipMemcpyDeviceToHost));
    same(got, dq_ref, xb, "nvfp4_dequant_unpack");
    HIP_OK(hipMemcpy(got, dy1, xb, hipMemcpyDeviceToHost));
    same(got, ob0_ref, xb, "nvfp4_observe_fake_quant y0");
    HIP_OK(hipMemcpy(got, dx, xb, hipMemcpyDeviceToHost));
    same(got, ob1_ref, xb, "nvfp4_observe_fake_quant y1 (in place)");

    HIP_OK(hipMemcpy(sc, scal, sizeof sc, hipMemcpyDeviceToHost));
    if (bits(sc[0]) != bits(a) || bits(sc[1]) != bits(a) || bits(sc[3]) != bits(a)) {
        fprintf(stderr, "amax: %08x %08x %08x, want %08x\n", bits(sc[0]), bits(sc[1]), bits(sc[3]), bits(a));
        failures++;
    }
    if (bits(sc[2]) != bits(g_ref)) {
        fprintf(stderr, "global scale %08x, want %08x\n", bits(sc[2]), bits(g_ref));
        failures++;
    }
    if (bits(sc[4]) != bits(st0_ref) || bits(sc[5]) != bits(st1_ref)) {
        fprintf(stderr, "observer states %08x %08x, want %08x %08x\n", bits(sc[4]), bits(sc[5]),
                bits(st0_ref), bits(st1_ref));
        failures++;
    }

    /* a call that must fail validation (a misaligned output) and enqueue nothing */
    if (nvfp4_fake_quant(dx, (char*)dx + 2, rows, cols, NULL, scal, s) != NVFP4_ERR_ALIGN) {
        fprintf(stderr, "a misaligned output was not rejected\n");
        failures++;
    }

    HIP_OK(hipStreamDestroy(s));
    void* bufs[] = {dx, dy, dy1, dp, ds, scal, ws};
    for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; i++)
        HIP_OK(hipFree(bufs[i]));
    free(x); free(fq_ref); free(p_ref); free(s_ref); free(dq_ref); free(ob0_ref); free(ob1_ref);
    free(got); free(gotp); free(gots);
    if (failures) {
        printf("%d mismatches\n", failures);
        return 1;
    }
    printf("%lldx%lld: all bit-exact\n", (long long)rows, (long long)cols);
    return 0;
}
