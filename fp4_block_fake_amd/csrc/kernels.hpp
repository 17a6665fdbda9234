// The streaming kernels of libnvfp4: amax, fake-quant, quantize-pack, dequant-unpack
// (whole-block and ragged rows), and the observer steps (included by nvfp4.hip).

#ifndef NVFP4_KERNELS_HPP
#define NVFP4_KERNELS_HPP

#include "device.hpp"

namespace {

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

// ---------------------------------------------------------------- ragged rows
//
// Rows whose length is not a multiple of 16 keep the half-block lanes of the
// whole-block kernels, over the zero-padded rows: padded half j is half
// hr = j - r hpr of row r = j / hpr (hpr = 2 ceil(cols / 16) halves per padded
// row), elements 8 hr .. 8 hr + 7 of the row, of which the first
// n = min(8, cols - 8 hr) exist (the rest are padding zeros).  Codes and scales
// keep the padded layout (dword j of the codes, scale byte j / 2), exactly as for
// whole-block rows.
//   Even lengths: a half starts on an even element, so it is four dwords, each
//   loaded and stored whole when it lies in the row.
//   Odd lengths (Odd): every other row starts on an odd element, so a half is
//   eight bf16 elements, each loaded and stored on its own (two lanes never
//   write into one dword).
// The bf16 side uses ordinary (allocating) loads and stores: a lane's accesses at
// a 16-byte lane stride each touch every line of the wave's span, and it is the
// L2 that merges them into whole lines.
struct HalfRows {
    const uint16_t* x;      // the tensor (16-byte aligned)
    int64_t cols;           // elements per row
    uint32_t hpr;           // halves per padded row
    int64_t nhalves;        // rows * hpr, below 2^32
};

// Element index of the first element of padded half j, and its count of real elements.
__device__ __forceinline__ int64_t row_half(const HalfRows& g, int64_t j, int& n)
{
    const uint32_t r = (uint32_t)j / g.hpr;
    const uint32_t hr = (uint32_t)j - r * g.hpr;
    const int64_t left = g.cols - 8 * (int64_t)hr;
    n = left < 8 ? (int)left : 8;
    return (int64_t)r * g.cols + 8 * (int64_t)hr;
}

// Whole halves move as one 16-byte access wherever the row puts them on a 4-byte
// boundary (global memory takes 16-byte accesses at any dword alignment); a half
// that starts on an odd element (odd lengths, every other row) moves as the
// aligned 16 bytes before its last element plus that element, and is stored as
// its first element, 12 aligned bytes and its last element.  Each half writes
// exactly its own bytes, so lanes never write into one dword.  A row's last,
// partial half moves element by element (dword by dword for even lengths).
struct __attribute__((aligned(4))) Dwords4 {
    uint32_t v[4];
};
struct __attribute__((aligned(4))) Dwords3 {
    uint32_t v[3];
};

// The n real elements of the half at element e, as four dwords (zeros past them).
template <bool Odd>
__device__ __forceinline__ void load_row_half(const uint16_t* x, int64_t e, int n, uint32_t (&w)[4])
{
    if (n == 8 && !(Odd && (e & 1))) {
        const Dwords4 d = *reinterpret_cast<const Dwords4*>(x + e);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w[i] = d.v[i];
    } else if (n == 8) {
        // elements e - 1 .. e + 6 from the dword boundary before e, then e + 7
        const Dwords4 d = *reinterpret_cast<const Dwords4*>(x + e - 1);
        const uint32_t last = x[e + 7];
        w[0] = __builtin_amdgcn_alignbit(d.v[1], d.v[0], 16);
        w[1] = __builtin_amdgcn_alignbit(d.v[2], d.v[1], 16);
        w[2] = __builtin_amdgcn_alignbit(d.v[3], d.v[2], 16);
        w[3] = (d.v[3] >> 16) | (last << 16);
    } else if (!Odd) {
        // a partial half of an even length has 2, 4 or 6 elements
        const uint32_t* xd = reinterpret_cast<const uint32_t*>(x) + e / 2;
#pragma unroll
        for (int i = 0; i < 3; ++i)
            w[i] = 2 * i < n ? xd[i] : 0u;
        w[3] = 0u;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = 2 * i < n ? x[e + 2 * i] : 0u;
            const uint32_t hi = 2 * i + 1 < n ? x[e + 2 * i + 1] : 0u;
            w[i] = lo | (hi << 16);
        }
    }
}

// The first n of the eight bf16 outputs o of a half to element e of y.
template <bool Odd>
__device__ __forceinline__ void store_row_half(uint16_t* y, int64_t e, int n, const uint4& o)
{
    const uint32_t v[4] = {o.x, o.y, o.z, o.w};
    if (n == 8 && !(Odd && (e & 1))) {
        Dwords4 d;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            d.v[i] = v[i];
        *reinterpret_cast<Dwords4*>(y + e) = d;
    } else if (n == 8) {
        Dwords3 d;
        d.v[0] = __builtin_amdgcn_alignbit(v[1], v[0], 16);
        d.v[1] = __builtin_amdgcn_alignbit(v[2], v[1], 16);
        d.v[2] = __builtin_amdgcn_alignbit(v[3], v[2], 16);
        y[e] = (uint16_t)(v[0] & 0xFFFFu);
        *reinterpret_cast<Dwords3*>(y + e + 1) = d;
        y[e + 7] = (uint16_t)(v[3] >> 16);
    } else if (!Odd) {
        uint32_t* yd = reinterpret_cast<uint32_t*>(y) + e / 2;
#pragma unroll
        for (int i = 0; i < 3; ++i)
            if (2 * i < n)
                yd[i] = v[i];
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (2 * i < n)
                y[e + 2 * i] = (uint16_t)(v[i] & 0xFFFFu);
            if (2 * i + 1 < n)
                y[e + 2 * i + 1] = (uint16_t)(v[i] >> 16);
        }
    }
}

// A quantizing pass over the padded halves with a grid stride, as quantize_pass:
// body(w, j, e, n) gets the four dwords of half j (zeros past the row), the element
// index e of its first element and its element count n.
template <bool Odd, bool Fence, typename Build, typename Body>
__device__ __forceinline__ void rows_pass(const HalfRows& g, Build build, Body body)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads * kUnroll;
    if (Fence)
        __builtin_amdgcn_sched_barrier(0);
    build();
    __syncthreads();
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

template <bool Partials, bool Odd>
__global__ __launch_bounds__(kThreads) void k_fake_quant_rows(HalfRows g, uint16_t* y, AmaxIn src)
{
    __shared__ uint4 table[128 * kEntryWords / 4];
    uint32_t* tab = reinterpret_cast<uint32_t*>(table);
    const AmaxOfPass<Partials> am(src);
    float gs = Partials ? 0.0f : global_scale_of(am.direct);
    rows_pass<Odd, Partials>(g, [&] {
        if (Partials)
            gs = global_scale_of(am.finish(src));
        build_table(gs, tab);
    }, [&](const uint32_t (&w)[4], int64_t, int64_t e, int n) {
        const uint32_t* t = tab + scale_byte_of(pair_max(w), gs) * kEntryWords;
        store_row_half<Odd>(y, e, n, decode_half(half_codes(w, t), __uint_as_float(t[1])));
    });
}

template <bool Partials, bool Odd>
__global__ __launch_bounds__(kThreads) void k_quantize_pack_rows(HalfRows g, uint32_t* __restrict__ packed,
                                                                 uint8_t* __restrict__ scales,
                                                                 float* __restrict__ gs_out, AmaxIn src)
{
    __shared__ uint4 table[128 * kEntryWords / 4];
    uint32_t* tab = reinterpret_cast<uint32_t*>(table);
    const AmaxOfPass<Partials> am(src);
    float gs = Partials ? 0.0f : global_scale_of(am.direct);
    if (!Partials && blockIdx.x == 0 && threadIdx.x == 0)
        *gs_out = gs;
    rows_pass<Odd, Partials>(g, [&] {
        if (Partials) {
            gs = global_scale_of(am.finish(src));
            if (blockIdx.x == 0 && threadIdx.x == 0)
                *gs_out = gs;
        }
        build_table(gs, tab);
    }, [&](const uint32_t (&w)[4], int64_t j, int64_t, int) {
        const uint32_t sb = scale_byte_of(pair_max(w), gs);
        store4<NVFP4_QP_NT_ST != 0>(packed + j, half_codes(w, tab + sb * kEntryWords));
        if (!(j & 1))
            scales[j >> 1] = (uint8_t)sb;
    });
}

template <bool Odd>
__global__ __launch_bounds__(kThreads) void k_dequant_unpack_rows(const uint32_t* __restrict__ packed,
                                                                  const uint8_t* __restrict__ scales,
                                                                  const float* __restrict__ gs_in,
                                                                  uint16_t* __restrict__ y, HalfRows g)
{
    __shared__ float sd_of[128];
    const float gs = *gs_in;
    if (threadIdx.x < 128)
        sd_of[threadIdx.x] = e4m3_decode(threadIdx.x) / gs;
    __syncthreads();
    const int64_t stride = (int64_t)gridDim.x * kThreads * kDqUnroll;
    for (int64_t base = (int64_t)blockIdx.x * kThreads * kDqUnroll + threadIdx.x; base < g.nhalves;
         base += stride) {
        uint32_t p[kDqUnroll], sc[kDqUnroll];
#pragma unroll
        for (int u = 0; u < kDqUnroll; ++u) {
            const int64_t j = base + (int64_t)u * kThreads;
            p[u] = j < g.nhalves ? packed[j] : 0u;
            sc[u] = j < g.nhalves ? scales[j >> 1] : 0u;
        }
#pragma unroll
        for (int u = 0; u < kDqUnroll; ++u) {
            const int64_t j = base + (int64_t)u * kThreads;
            if (j < g.nhalves) {
                int n;
                const int64_t e = row_half(g, j, n);
                store_row_half<Odd>(y, e, n, decode_half(p[u], sd_of[sc[u] & 0x7Fu]));
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

}  // namespace

#endif  // NVFP4_KERNELS_HPP
