// Launch shapes, cache hints and constants of libnvfp4 (included by nvfp4.hip).

#ifndef NVFP4_CONFIG_HPP
#define NVFP4_CONFIG_HPP

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
#define NVFP4_DQ_UNROLL 2         // half blocks per lane per iteration: unpack
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
// Tensors below NVFP4_MID_BYTES get fewer quantizing workgroups per CU: each
// then covers a few iterations (fewer table builds), 2-4 us faster on 64-112 MB
// tensors and slower on the 470 MB one.  Swept per pass (one process, 5-24 per
// CU): fake-quant was fastest at 7 (c4 activation 30.5 us against 31.3 at 8,
// c4 weight 52.6 against 53.2), quantize-pack at 8 (c4 weight 40.9 against
// 42.3 at 7); the two-output pass (dual fake-quant, observe step) at 6 or 16-32
// (41.0-41.4 us against 42.9-44.0 at 8 and 12: at 8 every workgroup of the
// c4 activation runs exactly two iterations in lockstep).
#ifndef NVFP4_MID_BYTES
#define NVFP4_MID_BYTES (256LL << 20)
#endif
#ifndef NVFP4_FQ_MID_WG_PER_CU
#define NVFP4_FQ_MID_WG_PER_CU 7
#endif
#ifndef NVFP4_QP_MID_WG_PER_CU
#define NVFP4_QP_MID_WG_PER_CU 8
#endif
#ifndef NVFP4_DUAL_MID_WG_PER_CU
#define NVFP4_DUAL_MID_WG_PER_CU 16
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
#ifndef NVFP4_TILE_XCD_REMAP
#define NVFP4_TILE_XCD_REMAP 1    // 1: the tiled linear groups each weight tile's x tiles on one XCD
#endif
#ifndef NVFP4_LIN_LDS_M
#define NVFP4_LIN_LDS_M 257       // rows of x from which the linear layer runs 256 x 256 LDS-staged tiles
#endif
#ifndef NVFP4_LIN_LDS_SMALL_M
#define NVFP4_LIN_LDS_SMALL_M 65   // rows of x from which the 128 x 128 LDS-staged tile is used
#endif
#ifndef NVFP4_LIN_LDS_PIPE
#define NVFP4_LIN_LDS_PIPE 1      // 1: the 4-wave LDS tile reads slice q + 1's operands before slice q's MFMAs
#endif
#ifndef NVFP4_LIN_LDS_FLAT
#define NVFP4_LIN_LDS_FLAT 1      // 1: whole groups of four K steps run without per-step branches
#endif
#ifndef NVFP4_LIN_LDS_KG2
#define NVFP4_LIN_LDS_KG2 1       // 1: the 128 x 128 LDS tile runs two K groups of 4 waves (K / 64 even)
#endif
#ifndef NVFP4_LIN_LDS_BUF
#define NVFP4_LIN_LDS_BUF 1       // 1: the LDS-staged linear kernel loads through buffer resources
#endif
#ifndef NVFP4_LIN_RETILE
#define NVFP4_LIN_RETILE 1        // 1: a partial last round of 256 x 256 linear tiles runs as narrower tiles
#endif
#ifndef NVFP4_LIN_NARROW
#define NVFP4_LIN_NARROW 1        // 1: 129-256 rows of x whose 128 x 128 tiles exceed the CUs run as 256 x 128 tiles
#endif
#ifndef NVFP4_LIN_RETILE_CUS
#define NVFP4_LIN_RETILE_CUS 0    // CUs the re-tiling and 256 x 128 tiles plan for; 0: the device's (a test build sets a few)
#endif
#ifndef NVFP4_LIN_LDS_REMAP
#define NVFP4_LIN_LDS_REMAP 1     // 1: the LDS-staged linear kernel orders its tiles by XCD
#endif
#ifndef NVFP4_TILE_DEPTH
#define NVFP4_TILE_DEPTH 6        // K steps of weight loads in flight per tiled-linear wave (even)
#endif
// Unpack: 2 half blocks per lane and up to 256 workgroups per CU, which gives the
// c5 weight one iteration per workgroup.  Measured in the c5 bench step (one
// process): the unpack 104.4 -> 94.0 us against 8 half blocks and 32 per CU, whose
// workgroups ran 1.75 iterations each; 1 or 4 half blocks, or fewer workgroups,
// were slower (97.7-110 us).
#ifndef NVFP4_DQ_WG_PER_CU
#define NVFP4_DQ_WG_PER_CU 256
#endif
// Workgroups per CU of the MXFP4 passes (one pass each, no per-workgroup table, so
// nothing to amortize): 256 gives the c5 weight one iteration per workgroup.
// Measured on c5 (warm loops, one process), 32 -> 256: fake-quant 157.2 -> 152.2 us,
// quantize-pack 110.7 -> 106.1, unpack 88.4 -> 85.6.
#ifndef NVFP4_MX_WG_PER_CU
#define NVFP4_MX_WG_PER_CU 256
#endif
// 1: the MXFP4 quantize-pack stores its fp32 block scales with non-temporal stores,
// as it does its codes.  c5 weight, loop of packs (one process): 103.2 -> 96.9 us,
// the copy stream's rate for its bytes.  (The same for the NVFP4 scale bytes slowed
// the c5 step: the unpack after the pack then reads them from HBM, 93.8 -> 95.8 us.)
#ifndef NVFP4_MX_SC_NT
#define NVFP4_MX_SC_NT 1
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
// Ragged rows of fewer blocks than this take the half-block kernels (their half
// index is 32-bit), larger ones the one-lane-per-block kernels.  A test build sets
// 0 to run every ragged shape through the latter.
#ifndef NVFP4_HALF_ROWS_MAX_BLOCKS
#define NVFP4_HALF_ROWS_MAX_BLOCKS (1LL << 31)
#endif
// 2 builds a test library in which every wave computes its codes from the
// correctly rounded quotient (the path that waves holding a block with an
// uncertified scale byte take), under every scale byte.
#ifndef NVFP4_EXACT_PATH
#define NVFP4_EXACT_PATH 1
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

}  // namespace

#endif  // NVFP4_CONFIG_HPP
