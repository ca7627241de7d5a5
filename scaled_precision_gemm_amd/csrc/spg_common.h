// Internal declarations and device helpers of the gfx950 library.
// Not part of the public ABI (include/spg.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/spg.h"

#define SPG_EXPORT extern "C" __attribute__((visibility("default")))

namespace spg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// Number formats
// ---------------------------------------------------------------------------

// binary32 -> E4M3FN code: round to nearest even, saturate at +-448, keep
// the sign of zero.  Integer rounding on the binary32 bit pattern: the three
// kept mantissa bits are rounded with the usual (half - 1 + lsb) increment;
// below the smallest normal (2^-6) the value is a multiple of 2^-9 and
// rint(|v| * 2^9) (exact scaling, round-half-even) gives the code directly.
__device__ __forceinline__ uint32_t encode_e4m3(float v)
{
    // All three cases are computed and one is selected: per-element branches
    // would diverge inside a wave.
    const uint32_t u = __float_as_uint(v);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    const uint32_t normal = ((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - ((127u - 7u) << 3);
    // (clamped so the float -> integer conversion stays in range when unused)
    const uint32_t sub = (uint32_t)__builtin_rintf(fminf(__uint_as_float(a) * 512.0f, 512.0f));   // |v| < 2^-6
    uint32_t code = a < 0x3C800000u ? sub : normal;
    code = a >= 0x43E00000u ? 0x7Eu : code;                                          // |v| >= 448
    return sign | code;
}

// binary32 -> E2M1 code (4 bits): nearest even, saturate at +-6, sign kept.
// The NVFP4 quantizers round with v_cvt_scalef32_pk_fp4_f32 instead, which
// was checked against this definition for every non-NaN binary32 value.
__device__ __forceinline__ uint32_t encode_e2m1(float v)
{
    const uint32_t u = __float_as_uint(v);
    const uint32_t sign = (u >> 28) & 0x8u;
    const uint32_t a = u & 0x7FFFFFFFu;
    const uint32_t normal = ((a + 0x1FFFFFu + ((a >> 22) & 1u)) >> 22) - ((127u - 1u) << 1);
    const uint32_t sub = (uint32_t)__builtin_rintf(fminf(__uint_as_float(a) * 2.0f, 16.0f));   // |v| < 1: halves
    uint32_t code = a < 0x3F800000u ? sub : normal;
    code = a >= 0x40C00000u ? 7u : code;                                            // |v| >= 6
    return sign | code;
}

// E4M3FN code -> binary32 (exact).  Codes 0x7F/0xFF (NaN) are never produced
// by the quantizers and are not decoded specially.
__device__ __forceinline__ float decode_e4m3(uint32_t c)
{
    uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
    float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
    return (c & 0x80u) ? -mag : mag;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// binary32 -> bf16 bits, round to nearest even (finite inputs; NaN kept NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------------------
// Wavefront (64 lanes) reductions
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
        v = v > o ? v : o;
    }
    return v;
}

// ---------------------------------------------------------------------------
// Host-side launchers shared between translation units
// ---------------------------------------------------------------------------
// Division by a launch constant d >= 1 for n < 2^31 as (umulhi(n, m) + n) >> s
// with s = ceil(log2 d), m = floor(2^32 (2^s - d) / d) + 1 (computed on the
// host): scalar multiply-high and shift instead of a division expanded on the
// vector unit.
struct FastDiv {
    uint32_t m, s;
};

// n / d for n < 2^31 with a FastDiv of d (multiply-high, add, shift).
__device__ __forceinline__ uint32_t fdiv_q(uint32_t n, const FastDiv &f) { return (__umulhi(n, f.m) + n) >> f.s; }

struct GemmArgs {
    void *out;
    const uint8_t *A;
    const uint8_t *W;
    const void *sa;
    const void *sw;
    const uint16_t *residual;
    int64_t M, N, K, batch;
    int64_t lda, ldw, ldo, ldr;
    int64_t stride_a, stride_w, stride_o, stride_r;
    int64_t sa_bstride, sw_bstride;   // batch stride of the scale arrays (elements)
    int32_t format, epilogue;
    const float *tscale_a, *tscale_w;
    float *partials;                  // split-K fp32 partial tiles (workspace)
    int32_t split_k;
    int64_t k_chunk;                  // K per split (multiple of the tile K)
    int64_t tiles_m, tiles_n;         // output tiles per product
    int64_t tile_begin, tile_count;   // the tiles this launch computes (of batch*tiles_m*tiles_n)
    FastDiv div_per, div_span, div_gm_last;   // by tiles_m*tiles_n, 8*tiles_n, tiles_m % 8
    uint64_t *clocks;                 // optional clock record (spg_gemm_desc.clock_probe), else null
    int32_t scale_layout;             // NVFP4 block-scale planes: SPG_SCALES_ROW_MAJOR or _BLOCKED
    int32_t bias_mode;                // ADD: 0 a residual matrix, 1 a bf16 bias row, 2 an E4M3 bias row
    const float *bias_scale;          // bias_mode 2: the bias row's fp32 scale
    // Output column segments (spg_out_split); nseg == 0: the one output
    // (out, ldo, stride_o).  Otherwise out / ldo hold segment 0 (every
    // segment is 16-byte aligned with ldo a multiple of 8, which is all the
    // alignment tests look at).  seg_b holds the segment boundaries in units
    // of 64 columns, 16 bits each (boundary i in bits 16 (i % 2) of word
    // i / 2).
    int32_t nseg;
    uint32_t seg_b[SPG_MAX_OUT_SPLITS / 2];
    struct Seg {
        uint16_t *out;
        int64_t ldo, stride, begin;
    } seg[SPG_MAX_OUT_SPLITS];
    // Half-height kernel: 0 - its work items are the two 128-row halves of
    // 256-row tiles tile_begin ..; 1 - the launch covers a grid of 128-row
    // tiles (tiles_m, the divisions and tile_count describe that grid)
    int32_t rows128;
};

// Output element (b, row, col) of a split output (nseg > 0) and the row
// stride of the segment holding it.  The segment's fields are loaded from the kernel-argument segment at an
// offset computed from col: the compiler cannot hoist such loads out of a
// persistent tile loop (read with constant indices, the whole table stayed
// in ~60 scalar registers across the main loop: the row-scaled ADD kernel's
// scalar spills grew from 194 to 282 and its tile by 7%), and unlike a
// run-time index into the argument itself this does not copy the arguments
// to scratch memory.  Every GEMM kernel takes one GemmArgs as its only
// argument, so it starts the kernel-argument segment.
__device__ __forceinline__ uint16_t *out_at(const GemmArgs &g, int64_t b, int64_t row, int64_t col, int64_t &ld)
{
    const uint32_t c64 = (uint32_t)(col >> 6);
    int s = 0;
#pragma unroll
    for (int i = 0; i + 1 < SPG_MAX_OUT_SPLITS; ++i)
        s += (i + 1 < g.nseg && c64 >= ((g.seg_b[i >> 1] >> (16 * (i & 1))) & 0xFFFFu)) ? 1 : 0;
    typedef const __attribute__((address_space(4))) GemmArgs::Seg *SegTable;
    const SegTable tab = (SegTable)((const __attribute__((address_space(4))) char *)__builtin_amdgcn_kernarg_segment_ptr() +
                                    offsetof(GemmArgs, seg));
    uint16_t *const out = tab[s].out;
    const int64_t l = tab[s].ldo, st = tab[s].stride, begin = tab[s].begin;
    ld = l;
    return out + (st ? b * st : 0) + row * l + (col - begin);
}

// Optional clock record of the main GEMM launch: thread 0 of workgroup 0
// stores the shader-clock counter and the 100 MHz reference counter when the
// kernel starts (which = 0) and ends (which = 1), at clocks[which] and
// clocks[2 + which].  Plain vector stores; nothing is kept live in between.
__device__ __forceinline__ void clock_mark(uint64_t *clocks, int which)
{
    if (clocks != nullptr && blockIdx.x == 0 && threadIdx.x == 0) {
        const uint64_t t = __builtin_amdgcn_s_memtime();
        const uint64_t r = __builtin_amdgcn_s_memrealtime();
        __builtin_nontemporal_store(t, clocks + which);
        __builtin_nontemporal_store(r, clocks + 2 + which);
    }
}

inline FastDiv make_fastdiv(uint32_t d)
{
    uint32_t sh = 0;
    while ((1ull << sh) < d) ++sh;
    return FastDiv{(uint32_t)((((1ull << sh) - d) << 32) / d + 1), sh};
}

hipError_t launch_gemm_fp8(const GemmArgs &g, const spg_plan &p, hipStream_t s);
hipError_t launch_gemm_fp8_half(const GemmArgs &g, hipStream_t s);   // tiles tile_begin.. as 128-row halves
hipError_t launch_gemm_nvfp4(const GemmArgs &g, const spg_plan &p, hipStream_t s);
// Products of at most 32 tokens: one workgroup per narrow_cols(epilogue)
// output columns (g.tiles_n column blocks per product) and batch entry.
// SWIGLU blocks carry 16 gate and 16 up rows; the others 32 weight rows, so
// each token fragment a wave reads serves two weight fragments (measured on
// 16 x 5120 x 17408: 20 us against 24 with 16 columns; the SwiGLU prefers
// 16: 37 against 44).
constexpr int narrow_cols(int epilogue) { return epilogue == SPG_EPI_SWIGLU ? 16 : 32; }
hipError_t launch_gemm_narrow(const GemmArgs &g, hipStream_t s);
hipError_t launch_splitk_reduce(const GemmArgs &g, int64_t tiles, hipStream_t s);
// [R, C] codes (row stride ld, batch stride bstride, 16-byte aligned rows)
// -> [C, R] with row stride R (R % 16 == 0), batch entries R * C apart.
hipError_t launch_transpose_u8(const uint8_t *src, int64_t R, int64_t C, int64_t ld, int64_t bstride,
                               int64_t batch, uint8_t *dst, hipStream_t s);
hipError_t launch_quantize_rowwise(const uint16_t *x, int64_t rows, int64_t K, int64_t ldx,
                                   uint8_t *q, int64_t ldq, float *scale, hipStream_t s);
hipError_t launch_quantize_tensor(const uint16_t *x, int64_t batch, int64_t rows, int64_t K,
                                  int64_t bstride, uint8_t *q, float *scale, uint32_t *ws,
                                  int64_t parts, hipStream_t s);
hipError_t launch_quantize_block16(const uint16_t *x, int64_t rows, int64_t K, uint8_t *q,
                                   uint8_t *bscale, float *tscale, int layout, bool single_launch, uint32_t *ws,
                                   int64_t parts, hipStream_t s);

// Workspace of quantize_block16: the single-launch path's sync area (its
// counters, flag and tensor scale on separate cache lines, then one maximum
// per block) in the first kBlock16SyncWords words, then the two-pass path's
// partial maxima.
constexpr int64_t kMaxFusedBlocks = 1024;
constexpr int64_t kBlock16SyncWords = 19 * 32 + kMaxFusedBlocks;

// Whether quantize_block16 runs as one launch on the current device.
bool quantize_block16_single_launch(int64_t rows, int64_t K);

// Partial-maximum blocks used by the per-tensor amax pass.
int64_t amax_parts(int64_t elems);

}  // namespace spg
