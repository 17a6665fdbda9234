// Test-only kernels (not part of libnvfp4): the gfx950 conversion instructions the
// library's kernels rely on, applied to every input of a range, so that
// tests/test_gpu_converters.py can compare each result with the CPU oracle.
//
//   which 0  v_cvt_scalef32_pk_fp4_f32, scale 1.0: binary32 pairs -> one byte of two
//            E2M1 codes (the element codes of the quantizing kernels)
//   which 1  v_cvt_pk_bf16_f32 (written as a float2 -> bf16x2 conversion, as the
//            library writes it): binary32 pairs -> two bf16 (every bf16 output)
//   which 2  v_cvt_pk_fp8_f32: binary32 -> E4M3 byte (the block scale byte)
//   which 3  v_cvt_scalef32_pk_f32_fp4, scale 1.0: every byte of codes under every
//            byte selector -> two binary32 values (decoding codes to values)
//
// Inputs are the binary32 bit patterns first, first + 1, ..., first + n - 1 (n even),
// made from the thread index, so the kernels read no memory.  Every thread writes
// only its own output slot, inside a buffer sized for exactly n inputs.
// Build: hipcc --offload-arch=gfx950 -O2 -ffp-contract=off -fPIC -shared.

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void k_fp4(uint32_t first, uint64_t pairs, uint8_t* out)
{
    const uint64_t p = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    if (p >= pairs)
        return;
    const uint32_t b0 = first + (uint32_t)(2 * p);
    const uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, __uint_as_float(b0), __uint_as_float(b0 + 1u),
                                                                1.0f, 0);
    out[p] = (uint8_t)(r & 0xFFu);
}

__global__ __launch_bounds__(kThreads) void k_bf16(uint32_t first, uint64_t pairs, uint32_t* out)
{
    const uint64_t p = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    if (p >= pairs)
        return;
    const uint32_t b0 = first + (uint32_t)(2 * p);
    const f32x2 v = {__uint_as_float(b0), __uint_as_float(b0 + 1u)};
    out[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__global__ __launch_bounds__(kThreads) void k_fp8(uint32_t first, uint64_t pairs, uint16_t* out)
{
    const uint64_t p = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
    if (p >= pairs)
        return;
    const uint32_t b0 = first + (uint32_t)(2 * p);
    const uint32_t r = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(b0), __uint_as_float(b0 + 1u), 0, false);
    out[p] = (uint16_t)(r & 0xFFFFu);
}

// 256 bytes x 4 selectors; the other three bytes of the source word hold a
// different pattern, so a wrong selector shows.
__global__ __launch_bounds__(kThreads) void k_fp4_decode(float* out)
{
    const uint32_t byte = threadIdx.x;                // one workgroup of 256 threads
    const uint32_t filler = (byte ^ 0x5Au) * 0x01010101u;
    f32x2 v[4];
    v[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((filler & ~0x000000FFu) | byte, 1.0f, 0);
    v[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((filler & ~0x0000FF00u) | (byte << 8), 1.0f, 1);
    v[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((filler & ~0x00FF0000u) | (byte << 16), 1.0f, 2);
    v[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((filler & ~0xFF000000u) | (byte << 24), 1.0f, 3);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        out[(s * 256 + byte) * 2] = v[s].x;
        out[(s * 256 + byte) * 2 + 1] = v[s].y;
    }
}

}  // namespace

// Runs converter `which` over n inputs from bit pattern `first` (n even, n <= 2^28)
// and copies the results to host memory at `host_out`:
//   which 0: n / 2 bytes; 1: n uint16; 2: n bytes; 3: (first, n ignored) 2048 floats.
// Returns 0, or the HIP error code.
extern "C" int conv_run(int which, uint32_t first, uint64_t n, void* host_out)
{
    if (which < 0 || which > 3 || (which != 3 && (n == 0 || n % 2 != 0 || n > (1ull << 28))))
        return (int)hipErrorInvalidValue;
    if (which != 3 && (uint64_t)first + n > (1ull << 32))
        return (int)hipErrorInvalidValue;
    const uint64_t pairs = n / 2;
    const size_t bytes = which == 0 ? pairs : which == 1 ? 2 * n : which == 2 ? n : 2048 * sizeof(float);
    void* d = nullptr;
    hipError_t e = hipMalloc(&d, bytes);
    if (e != hipSuccess)
        return (int)e;
    const unsigned grid = (unsigned)((pairs + kThreads - 1) / kThreads);
    switch (which) {
    case 0: k_fp4<<<grid, kThreads>>>(first, pairs, static_cast<uint8_t*>(d)); break;
    case 1: k_bf16<<<grid, kThreads>>>(first, pairs, static_cast<uint32_t*>(d)); break;
    case 2: k_fp8<<<grid, kThreads>>>(first, pairs, static_cast<uint16_t*>(d)); break;
    default: k_fp4_decode<<<1, 256>>>(static_cast<float*>(d)); break;
    }
    e = hipGetLastError();
    if (e == hipSuccess)
        e = hipMemcpy(host_out, d, bytes, hipMemcpyDeviceToHost);
    const hipError_t f = hipFree(d);
    return (int)(e != hipSuccess ? e : f);
}
