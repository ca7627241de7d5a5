// Pieces shared by the FP8 and NVFP4 GEMM kernels: tile scheduling, the LDS
// layout of a K stage, the accumulator layout, split-K partial stores and the
// fused bf16 epilogues.
//
// Both kernels use a 256 x 256 workgroup tile computed by 4 waves (2 x 2),
// each wave a 128 x 128 sub-tile of 4 x 4 32x32 MFMA blocks.  The 32x32 MFMA
// result layout is the same for every input format: lane l, register e of a
// block holds row (e / 4) * 8 + (l / 32) * 4 + (e % 4), column l % 32 of the
// block, rows coming from the first MFMA operand.  The kernels pass the W
// fragment first, so a block's rows are W rows (output columns) and its
// columns are A rows (tokens): each lane owns four consecutive output columns
// of one token row per group of four registers, which leave as one 8-byte
// store straight from registers.
#pragma once

#include "spg_common.h"

namespace spg {
namespace gemm {

constexpr int kBM = 256, kBN = 256, kThreads = 256;
constexpr int kRowBytes = 128;                 // one LDS row of a K stage
constexpr int kStageBytes = kBM * kRowBytes;   // one operand, one stage
constexpr int kGroupM = 8;                     // tile-rows per raster group

// Byte offset of 16-byte chunk `chunk` (0..7) of a 128-byte LDS row.  gfx950's
// LDS has 64 four-byte banks and serves a 16-byte-per-lane access for 16
// lanes per clock (256 bytes).  Sixteen consecutive rows read at the same
// logical chunk cover rows of both parities; XOR-ing the chunk with
// (row >> 1) & 7 gives the eight rows of each parity eight distinct 16-byte
// bank groups, so the 16 lanes touch all 64 banks once (measured: the same
// rate as a contiguous read; XOR with row & 7 measures half that).  Stage
// buffers are aligned to the pattern's 2 KiB period.
__device__ __forceinline__ uint32_t swz(uint32_t row, uint32_t chunk)
{
    return row * kRowBytes + ((chunk ^ ((row >> 1) & 7u)) << 4);
}

// Workgroup id -> tile id so that each XCD (ids congruent mod 8, which the
// dispatcher places round-robin) gets one contiguous range of tile ids.
__device__ __forceinline__ int64_t xcd_remap(int64_t wg, int64_t nwg)
{
    const int64_t q = nwg / 8, r = nwg % 8;
    const int64_t xcd = wg % 8, idx = wg / 8;
    const int64_t base = xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q;
    return base + idx;
}

// ---- direct-to-LDS copies and explicit waits (shared by the GEMM kernels) ----
constexpr uint32_t kOOB = 0x80000000u;        // buffer offset past any range

// Raw buffer resource: base, no stride, `bytes` in range, dword format bits.
__device__ __forceinline__ v4i make_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t b = (uint64_t)base;
    v4i r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = 0x00020000;
    return r;
}

// 16 bytes per lane from rsrc + voff + soff into LDS at lds_base + 16 * lane.
// Issued as inline assembly so the compiler does not treat every later LDS
// read as dependent on it; completion is awaited explicitly (vmcnt) before
// the barrier that publishes the stage.
__device__ __forceinline__ void dma16(uint32_t lds_base, uint32_t voff, v4i rsrc, uint32_t soff)
{
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(lds_base), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}

// 4 bytes per lane from rsrc + voff + soff into LDS at lds_base + 4 * lane
// (same rules as dma16).
__device__ __forceinline__ void dma4(uint32_t lds_base, uint32_t voff, v4i rsrc, uint32_t soff)
{
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :: "s"(lds_base), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void block_barrier()
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Lane index 0..63 recomputed from the execution mask (full at every call
// site): cheaper for the register allocator than keeping threadIdx.x alive,
// whose spill reload would wait on every outstanding memory operation.
// (volatile assembly: the builtins would be computed once and spilled).
__device__ __forceinline__ int lane_id()
{
    int r;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(r));
    return r;
}

// silu(g) * u = g / (1 + exp(-g)) * u with the hardware exp2 and reciprocal
// (about 1 ulp each; the SwiGLU output tolerance is 2^-8 relative), the
// denominator carried as d = (1 + exp(-g)) 2^-64 and the 2^-64 given back
// as 2^-32 on each factor: y = (g / d 2^-32) (u 2^-32).  Unscaled, from
// g = -87.3 the reciprocal of the denominator is subnormal (the hardware
// reciprocal flushes it to zero) and from g = -88.7 exp(-g) overflows, so
// silu(g) u came out 0 where it can still be a normal bf16 value (g = -88,
// u = -46: 1.8e-35).  Scaled, 1 / d stays normal down to g = -131 (exp(-g)
// 2^-64 is finite down to -133); g / d 2^-32 = silu(g) 2^32 is normal down
// to g = -113, and u 2^-32 is normal for |u| > 2^-94, so the product is
// right wherever it is a normal number, up to fp32's largest (below
// g = -113 silu(g) u is under 2^-126 for any |u| < 2^36), for gates below
// 2^64: g / d, formed first, is g 2^64 for large g and passes fp32's range
// there.  Against the unscaled form this costs two multiplies; the
// offset in the exponent argument costs 2^-18 of absolute precision in it
// (a relative 2^-18 in exp).
__device__ __forceinline__ float swiglu_f32(float g, float u)
{
    const float d = __builtin_amdgcn_exp2f(__builtin_fmaf(g, -1.44269504f, -64.0f)) + 0x1p-64f;
    return (g * __builtin_amdgcn_rcpf(d) * 0x1p-32f) * (u * 0x1p-32f);
}

struct Tile {
    int64_t global;   // tile id over the whole batch (split-K bookkeeping)
    int64_t b;        // batch entry
    int64_t m0;       // first output row
    int64_t tn;       // tile column index
    int64_t n0;       // first W row (SWIGLU: first gate row; up rows at N/2 + n0)
    int64_t c0;       // first output column
};

// Tiles of one product are rasterized in groups of kGroupM tile-rows,
// column-major inside a group, so neighbouring tile ids share A panels
// (same rows) and W panels (same columns) through the L2 of their XCD.
__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv &f) { return fdiv_q(n, f); }

// All in 32-bit scalar arithmetic (tile counts are below 2^31).
template <int EPI, int ROWS = kBM>
__device__ __forceinline__ Tile tile_from_id(const GemmArgs &g, int64_t t)
{
    Tile T;
    T.global = t;
    const uint32_t tt = (uint32_t)t, tiles_m = (uint32_t)g.tiles_m, tiles_n = (uint32_t)g.tiles_n;
    const uint32_t b = fdiv(tt, g.div_per);
    const uint32_t rem = tt - b * (tiles_m * tiles_n);
    const uint32_t grp = fdiv(rem, g.div_span);
    const uint32_t first_m = grp * kGroupM;
    const uint32_t tin = rem - grp * (kGroupM * tiles_n);
    const uint32_t gm = min((uint32_t)kGroupM, tiles_m - first_m);
    const uint32_t tn = gm == (uint32_t)kGroupM ? tin / kGroupM : fdiv(tin, g.div_gm_last);
    T.b = b;
    T.m0 = (int64_t)(first_m + (tin - tn * gm)) * ROWS;
    T.tn = tn;
    T.n0 = EPI == SPG_EPI_SWIGLU ? (int64_t)tn * (kBN / 2) : (int64_t)tn * kBN;
    T.c0 = T.n0;
    return T;
}

// Work item of a launch over tile_count * split_k workgroups (1-D grid): the
// tile (counted from tile_begin) and its K slice.  Work ids run slice-major
// (all tiles of slice 0, then slice 1, ...) and each XCD takes one
// contiguous range of them, so the workgroups sharing an XCD's L2 mostly
// work on the same K slice of neighbouring tiles and share its A and W
// panels (ordering tiles first, slices last, would give every XCD all
// slices of fewer tiles: about twice the distinct panel bytes per XCD).
struct WorkItem {
    int64_t tile;
    int split;
};

__device__ __forceinline__ WorkItem work_item(const GemmArgs &g)
{
    const uint32_t n = (uint32_t)(g.tile_count * g.split_k);
    const uint32_t v = (uint32_t)xcd_remap(blockIdx.x, n);
    const uint32_t s = v / (uint32_t)g.tile_count;
    return WorkItem{(int64_t)(v - s * (uint32_t)g.tile_count), (int)s};
}

// W row of tile row r (0..255) and whether it exists.  SWIGLU: rows 0..127
// are gate rows n0 + r, rows 128..255 the matching up rows N/2 + n0 + r - 128.
template <int EPI>
__device__ __forceinline__ int64_t w_row(const GemmArgs &g, const Tile &T, int r, bool &ok)
{
    if (EPI == SPG_EPI_SWIGLU) {
        const int64_t Nh = g.N / 2, j = T.n0 + (r & 127);
        ok = j < Nh;
        return r < 128 ? j : Nh + j;
    }
    const int64_t j = T.n0 + r;
    ok = j < g.N;
    return j;
}

// acc[x][y]: W block x (tile rows wtile_row0(wn, x) ..+31) times A block y
// (tile rows wm * 128 + y * 32 ..+31) of wave (wm, wn).
using Acc = v16f[4][4];

__device__ __forceinline__ void zero_acc(Acc &acc)
{
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[x][y][e] = 0.0f;
}

// First W-tile row of W block x of a wave in column half wn.  SWIGLU: blocks
// 0,1 are gate rows and blocks 2,3 the matching up rows (tile rows 128 + the
// same offsets), so a gate value and its up partner sit in the same register
// of the same lane.
template <int EPI>
__device__ __forceinline__ int wtile_row0(int wn, int x)
{
    if (EPI == SPG_EPI_SWIGLU) return x < 2 ? wn * 64 + x * 32 : 128 + wn * 64 + (x - 2) * 32;
    return wn * 128 + x * 32;
}

// Scale factors of the tile, one entry per A-tile row (sa) and per W-tile
// row (sw); the epilogue forms acc * sa * sw.  Thread i supplies row i:
//   E4M3 per row:    sa = s_a[row], sw = s_w[W row]
//   E4M3 per tensor: sa = s_a, sw = s_w (of the batch entry)
//   NVFP4:           sa = 2^7 * tA, sw = 2^7 * tW (the two 2^7 undo the
//                    operand offsets of the kernel's f16 decode).  The
//                    tensor scales stay separate factors: each is at most
//                    bf16's maximum / 2688, so 2^7 t < 1.6e37, while their
//                    product can pass fp32's range for outputs that do not
template <int EPI, int SMODE>
__device__ __forceinline__ void scale_values(const GemmArgs &g, const Tile &T, float &va, float &vw)
{
    const int tid = threadIdx.x;
    if (SMODE == SPG_FMT_NVFP4) {
        va = 128.0f * *g.tscale_a;
        vw = 128.0f * *g.tscale_w;
    } else if (SMODE == SPG_FMT_E4M3_ROW) {
        bool wok;
        const int64_t wr = w_row<EPI>(g, T, tid, wok);
        const int64_t r = T.m0 + tid;
        const float *sa = (const float *)g.sa + (g.stride_a ? T.b * g.sa_bstride : 0);
        const float *sw = (const float *)g.sw + (g.stride_w ? T.b * g.sw_bstride : 0);
        va = r < g.M ? sa[r] : 0.0f;
        vw = wok ? sw[wr] : 0.0f;
    } else {
        va = ((const float *)g.sa)[g.stride_a ? T.b : 0];
        vw = ((const float *)g.sw)[g.stride_w ? T.b : 0];
    }
}

// The tile's scale factors into LDS.  Must be called by all kThreads
// threads; a barrier must follow before use.
template <int EPI, int SMODE>
__device__ __forceinline__ void stage_scales(const GemmArgs &g, const Tile &T, float *lds_sa, float *lds_sw)
{
    float va, vw;
    scale_values<EPI, SMODE>(g, T, va, vw);
    lds_sa[threadIdx.x] = va;
    lds_sw[threadIdx.x] = vw;
}

// Bias of output column col (< N) of batch entry b, for the ADD epilogue
// with a bias row: the bf16 value (bias_mode 1), or the E4M3 code times the
// bias scale, dequantized in fp32 (bias_mode 2; AstrAI commit log, the
// commit fusing the bias: FP8 bias storage dequantized after the operand
// scaling).
__device__ __forceinline__ float bias_at(const GemmArgs &g, int64_t b, int64_t col)
{
    const int64_t off = (g.stride_r ? b * g.stride_r : 0) + col;
    if (g.bias_mode == 1) return __uint_as_float((uint32_t)g.residual[off] << 16);
    return decode_e4m3(((const uint8_t *)g.residual)[off]) * *g.bias_scale;
}

// LDS floats a kernel with epilogue EPI provides for the bias of a bias row:
// 128 columns per wave (ADD), else a placeholder.
template <int EPI>
constexpr int bias_words() { return EPI == SPG_EPI_ADD ? 4 * 128 : 4; }

// Split-K, part 1: every K slice stores its fp32 partial tile and stops; a
// second kernel (splitk_reduce_kernel) sums the slices once all have
// finished - the kernel boundary orders the stores before the loads, so no
// device-scope fence or counter is needed.  Layout of one (tile, slice)
// partial, 65536 floats: element 4q + r (q, r = 0..3) of block b = 4x + y of
// thread i at (4b + q) * 1024 + 4i + r, so every store instruction of a wave
// writes 1 KiB of whole cache lines.  (Storing a thread's 16 elements
// contiguously instead made each instruction write 16 bytes into each of 32
// lines: the 61 MB of partials of 1024 x 5120 x 17408 in three slices then
// took ~45 us and the whole call 0.143 ms, against 0.095 ms now.)  Partial
// (t, s) of a launch starts at float (t * S + s) * 65536, t counted from
// tile_begin.
// Only token rows below M are stored (the reduction reads no others): with a
// few tokens per tile (decode widths) that is a small part of the tile.
__device__ __forceinline__ void splitk_store(const GemmArgs &g, const Tile &T, int split, const Acc &acc)
{
    float *base = g.partials + ((T.global - g.tile_begin) * g.split_k + split) * (int64_t)(kBM * kBN) + threadIdx.x * 4;
    const int64_t row_l = T.m0 + (int64_t)(threadIdx.x >> 7) * 128 + (threadIdx.x & 31);   // block y = 0
#pragma unroll
    for (int blk = 0; blk < 16; ++blk) {
        const v16f &a = acc[blk >> 2][blk & 3];
        if (row_l + (blk & 3) * 32 >= g.M) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *reinterpret_cast<v4f *>(base + (blk * 4 + q) * (kThreads * 4)) =
                v4f{a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
    }
}

typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Two binary32 -> two bf16 (round to nearest even) packed low-first in one
// dword (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{lo, hi}, v2bf));
}

struct EpiOut {
    uint16_t *out;            // output of the tile's batch entry
    const uint16_t *res;      // residual of the tile's batch entry (ADD)
    int64_t nvalid;           // output columns (N, or N/2 for SWIGLU)
    bool vec;                 // 8-byte output / residual accesses allowed
};

template <int EPI>
__device__ __forceinline__ EpiOut epi_out(const GemmArgs &g, const Tile &T)
{
    EpiOut o;
    o.out = (uint16_t *)g.out + (g.stride_o ? T.b * g.stride_o : 0);
    o.res = g.residual ? g.residual + (g.stride_r ? T.b * g.stride_r : 0) : nullptr;
    o.nvalid = EPI == SPG_EPI_SWIGLU ? g.N / 2 : g.N;
    o.vec = ((((uintptr_t)o.out) & 7) == 0) && ((g.ldo & 3) == 0);
    if (EPI == SPG_EPI_ADD && g.bias_mode == 0) o.vec = o.vec && ((((uintptr_t)o.res) & 7) == 0) && ((g.ldr & 3) == 0);
    return o;
}

// Fused epilogue of one 32x32 block straight from registers:
//   v = acc * lds_sa[token row] * lds_sw[W row]
//   STORE: bf16(v); ADD: bf16(v + residual), one rounding of the fp32 sum
//   (a bias row: v + the bias of the column, dequantized in fp32);
//   SWIGLU: bf16(silu(gate) * up), gate from `a`, up from `up` (same layout)
// Lane l writes token row wm * 128 + y * 32 + l % 32 of the tile and, per
// register group q, the four output columns at W-tile row
// w0 + 8 q + 4 (l / 32): one 8-byte store (2-byte stores at a ragged right
// edge or for outputs that are not 8-byte aligned).
template <int EPI>
__device__ __forceinline__ void epilogue_block(const GemmArgs &g, const Tile &T, const EpiOut &o, int w0, int y,
                                               const v16f &a, const v16f &up, const float *lds_sa,
                                               const float *lds_sw)
{
    const int lane = threadIdx.x & 63, wm = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) >> 1;
    const int l32 = lane & 31, khalf = lane >> 5;
    const int rl = wm * 128 + y * 32 + l32;
    const int64_t row = T.m0 + rl;
    if (row >= g.M) return;
    const float sa = lds_sa[rl];
    const uint16_t *rrow = EPI == SPG_EPI_ADD ? o.res + row * g.ldr : nullptr;
    const bool brow = EPI == SPG_EPI_ADD && g.bias_mode != 0;

    // residual (or bias) first, so its loads are in flight during the
    // arithmetic
    uint2 rv[4];
    float bv[EPI == SPG_EPI_ADD ? 4 : 1][4];
    if (EPI == SPG_EPI_ADD && brow) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t col = T.c0 + w0 + q * 8 + khalf * 4;
#pragma unroll
            for (int j = 0; j < 4; ++j) bv[EPI == SPG_EPI_ADD ? q : 0][j] = col + j < o.nvalid ? bias_at(g, T.b, col + j) : 0.0f;
        }
    } else if (EPI == SPG_EPI_ADD) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t col = T.c0 + w0 + q * 8 + khalf * 4;
            if (o.vec && col + 4 <= o.nvalid) {
                rv[q] = *reinterpret_cast<const uint2 *>(rrow + col);
            } else {
                uint32_t h[4] = {0, 0, 0, 0};
                for (int j = 0; j < 4; ++j)
                    if (col + j < o.nvalid) h[j] = rrow[col + j];
                rv[q] = make_uint2(h[0] | h[1] << 16, h[2] | h[3] << 16);
            }
        }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int wl = w0 + q * 8 + khalf * 4;
        const int64_t col = T.c0 + wl;
        const v4f sw = *reinterpret_cast<const v4f *>(lds_sw + wl);
        const v4f swu = EPI == SPG_EPI_SWIGLU ? *reinterpret_cast<const v4f *>(lds_sw + 128 + wl) : v4f{};
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = q * 4 + j;
            if (EPI == SPG_EPI_SWIGLU) {
                const float vg = a[e] * sa * sw[j];
                const float vu = up[e] * sa * swu[j];
                v[j] = swiglu_f32(vg, vu);
            } else {
                v[j] = a[e] * sa * sw[j];
            }
        }
        if (EPI == SPG_EPI_ADD && brow) {
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] += bv[EPI == SPG_EPI_ADD ? q : 0][j];
        } else if (EPI == SPG_EPI_ADD) {
            v[0] += bf16_lo(rv[q].x);
            v[1] += bf16_hi(rv[q].x);
            v[2] += bf16_lo(rv[q].y);
            v[3] += bf16_hi(rv[q].y);
        }
        const uint2 pk = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        if (col >= o.nvalid) continue;
        int64_t ld;
        uint16_t *const dst = g.nseg ? out_at(g, T.b, row, col, ld)   // a 4-column group never straddles segments
                                     : o.out + row * g.ldo + col;
        (void)ld;
        if (o.vec && col + 4 <= o.nvalid) {
            *reinterpret_cast<uint2 *>(dst) = pk;
        } else {
            const uint32_t w[2] = {pk.x, pk.y};
            for (int j = 0; j < 4 && col + j < o.nvalid; ++j) dst[j] = (uint16_t)(w[j >> 1] >> (16 * (j & 1)));
        }
    }
}

// Fused epilogue of the whole tile (no split), transposed through LDS so that
// the output leaves in whole rows.  Stores cost about one cycle per distinct
// cache line an instruction touches: in the accumulator layout one store
// instruction covers 32 token rows (32 lines), after the transpose it covers
// 8 whole 128-byte row segments (measured on 8192 x 8192 bf16: 3.3 TB/s for
// the former pattern, 6.5 TB/s for whole rows).
//
// Each wave works through its 128 x 128 quadrant (SWIGLU: 128 x 64 outputs)
// in passes of 32 token rows x 64 columns, staged in a private 4 KiB region,
// so no workgroup barrier is involved.  Row r of the region holds 128 bytes
// of token row (pass base + r); its 16-byte chunks are XOR-swizzled (chunk c
// at c ^ ((r >> 1) & 7)) so that both the fragment-order writes (one row per
// lane) and the row-order reads spread over all 64 banks.  Per pass:
//  1. ADD: the residual block is copied into the region row by row;
//  2. every lane forms v = acc * lds_sa * lds_sw (+ residual read back from
//     the region in fp32, one rounding; SWIGLU silu(gate) * up) and writes the
//     bf16 results in place (8 bytes per register group);
//     BIAS (ADD with a bias row): step 1 is skipped; each wave first stages
//     the fp32 biases of its 128 columns in its own 512 bytes of lds_bias,
//     and step 2 adds the bias of the column;
//  3. the region leaves as 16-byte chunks of whole 128-byte row segments.
// `region` is this wave's 4 KiB, 16-byte aligned, used by nothing else.
//
// STAGED (ADD with a residual matrix, FULL, and a caller that gives each
// wave one 4 KiB region per pass): step 1 is replaced by direct-to-LDS
// copies of every pass's residual block, all issued when the epilogue
// starts, each lane fetching the chunk that lands at its swizzled place.
// Row by row the residual costs one HBM round trip per pass; with every
// workgroup of a launch in its epilogue at once (one tile per workgroup)
// those round trips queue behind each other (measured on 4096 x 5120 x
// 6144 NVFP4: 61K cycles of a 340K-cycle tile).
constexpr int kEpiRegionBytes = 4 * 4096;   // per workgroup

// FULL: the wave's whole quadrant lies inside the output (and residual) and
// both are 16-byte aligned with row strides a multiple of 8 elements - no
// bounds checks or narrow-store paths, hence no per-store branches.
// MI: 32-row A blocks per wave (4; 2 in a half-height tile, whose waves
// hold acc[x][0..1] and cover token rows wm * 64 .. wm * 64 + 63).
// GIVEN: wave_in is the caller's wave index; otherwise it is derived here.
// SPLITOUT: the output is column segments (g.nseg > 0), addressed per pass.
template <int EPI, bool FULL, int MI = 4, bool GIVEN = false, bool BIAS = false, bool STAGED = false,
          bool SPLITOUT = false>
__device__ __forceinline__ void epilogue_impl(const GemmArgs &g, const Tile &T, const Acc &acc, const float *lds_sa,
                                              const float *lds_sw, float *lds_bias, uint8_t *region_base,
                                              int wave_in)
{
    uint8_t *const region = region_base;
    static_assert(!BIAS || EPI == SPG_EPI_ADD, "a bias row belongs to the ADD epilogue");
    static_assert(!STAGED || (EPI == SPG_EPI_ADD && FULL && !BIAS), "staged residual blocks: ADD, whole quadrants");
    constexpr bool SW = EPI == SPG_EPI_SWIGLU;
    constexpr int NP = SW ? 1 : 2;            // 64-column passes per 32-row block
    // opaque to the optimizer: lane-derived offsets are recomputed per call
    // instead of being hoisted (and spilled) across a persistent tile loop
    const int lane = lane_id();
    // the wave index is uniform: keeping it (and every row / column bound
    // derived from it) in scalar registers keeps the pass branches uniform
    const int wave = GIVEN ? wave_in : __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, khalf = lane >> 5;
    const EpiOut o = epi_out<EPI>(g, T);
    const bool vec16 = FULL || (((((uintptr_t)o.out) & 15) == 0) && ((g.ldo & 7) == 0));
    const bool rvec = FULL || (EPI == SPG_EPI_ADD && !BIAS && ((((uintptr_t)o.res) & 15) == 0) && ((g.ldr & 7) == 0));
    auto phys = [](int r, int c) -> int { return c ^ ((r >> 1) & 7); };
    const int rr = lane >> 3, rc = lane & 7;  // row-order lane position: 8 rows x 8 chunks
    // 32-bit element offsets inside a 32-row block (ldo, ldr < 2^26)
    const uint32_t ldo1 = (uint32_t)g.ldo, ldr = (uint32_t)g.ldr;

    // every scale factor this lane needs, read from LDS before any region
    // write (the compiler cannot move LDS reads across LDS writes it cannot
    // prove disjoint, so reading them per element would wait on each)
    // (BIAS: the column scales are read with the biases, next to their use,
    // which keeps the epilogue within the registers the tile loop leaves)
    float *const bias_w = lds_bias + (BIAS ? wave * 128 : 0);   // this wave's columns wn * 128 ..
    if (BIAS) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t c = T.c0 + wn * 128 + h * 64 + lane;
            bias_w[h * 64 + lane] = c < o.nvalid ? bias_at(g, T.b, c) : 0.0f;
        }
    }
    if (STAGED) {
        // every pass's residual block into its region (pass (y, p) at
        // region + (y * NP + p) * 4096): four 1 KiB copies of 8 rows each;
        // lane L of a copy fills row 8 i + L / 8, physical chunk L % 8, so it
        // fetches logical chunk (L % 8) ^ ((row >> 1) & 7).  Offsets are
        // relative to the quadrant's first element (caller: MI * 32 rows of
        // ldr elements span less than 2^31 bytes).
        const uint16_t *rb = o.res + (T.m0 + wm * (MI * 32)) * g.ldr + T.c0 + wn * 128;
        const v4i rs = make_rsrc(rb, (uint32_t)((int64_t)MI * 32 * g.ldr * 2));
        const uint32_t lbase = (uint32_t)__builtin_amdgcn_readfirstlane(
            (int)(uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)region);
#pragma unroll
        for (int y = 0; y < MI; ++y)
#pragma unroll
            for (int p = 0; p < NP; ++p)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t r = (uint32_t)(8 * i) + ((uint32_t)lane >> 3);
                    const uint32_t c = ((uint32_t)lane & 7u) ^ ((r >> 1) & 7u);
                    const uint32_t voff = (((uint32_t)(y * 32) + r) * ldr + (uint32_t)(p * 64) + c * 8u) * 2u;
                    dma16(lbase + (uint32_t)((y * NP + p) * 4096 + i * 1024), voff, rs, 0);
                }
        wait_vmem<0>();   // only this wave reads its regions
    }
    // ADD over whole quadrants: each pass's residual block is loaded during
    // the pass before (issued right after that pass's block reached the
    // region), so its round trip overlaps the conversion and the stores
    // instead of opening every pass
    constexpr bool PREF = EPI == SPG_EPI_ADD && !BIAS && !STAGED && FULL;
    v4i rpre[4];
    auto res_load = [&](int y, int p) {
        const uint16_t *rb = o.res + (T.m0 + wm * (MI * 32) + y * 32) * g.ldr + T.c0 + wn * 128 + p * 64;
#pragma unroll
        for (int it = 0; it < 4; ++it)
            rpre[it] = __builtin_nontemporal_load(
                reinterpret_cast<const v4i *>(rb + (uint32_t)((it * 8 + rr) * ldr + rc * 8)));   // read once
    };
    if (PREF) res_load(0, 0);
    constexpr int NX = SW ? 2 : 4;
    float sa_r[MI];
    v4f sw_r[BIAS ? 1 : NX][4], swu_r[SW ? 2 : 1][4];
#pragma unroll
    for (int y = 0; y < MI; ++y) sa_r[y] = lds_sa[wm * (MI * 32) + y * 32 + l32];
    if (!BIAS) {
#pragma unroll
        for (int x = 0; x < NX; ++x)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int wl = wtile_row0<EPI>(wn, x) + q * 8 + khalf * 4;
                sw_r[BIAS ? 0 : x][q] = *reinterpret_cast<const v4f *>(lds_sw + wl);
                if (SW) swu_r[x & 1][q] = *reinterpret_cast<const v4f *>(lds_sw + 128 + wl);
            }
    }

#pragma unroll
    for (int y = 0; y < MI; ++y) {
        const int64_t row0 = T.m0 + wm * (MI * 32) + y * 32;
        const int rows_valid = FULL ? 32 : (int)min((int64_t)32, g.M - row0);
        if (rows_valid <= 0) break;                                 // uniform per wave
        const float sa = sa_r[y];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            uint8_t *const region = region_base + (STAGED ? (y * NP + p) * 4096 : 0);
            const int64_t col0 = T.c0 + (SW ? wn * 64 : wn * 128 + p * 64);
            const int cols_valid = FULL ? 64 : (int)min((int64_t)64, o.nvalid - col0);
            if (cols_valid <= 0) break;                             // uniform per wave
            // keep each pass's work inside the pass (hoisting it all would
            // need more registers than the accumulators leave)
            __builtin_amdgcn_sched_barrier(0);
            int64_t ldo_p = 0;
            uint16_t *const obase = SPLITOUT ? out_at(g, T.b, row0, col0, ldo_p)   // one segment per 64 columns
                                             : o.out + row0 * g.ldo + col0;         // uniform
            const uint32_t ldo = SPLITOUT ? (uint32_t)ldo_p : ldo1;

            // 1. residual block -> region
            if (PREF) {
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const int r = it * 8 + rr;
                    *reinterpret_cast<v4i *>(region + r * 128 + phys(r, rc) * 16) = rpre[it];
                }
                if (p + 1 < NP)
                    res_load(y, p + 1);
                else if (y + 1 < MI)
                    res_load(y + 1, 0);
            } else if (EPI == SPG_EPI_ADD && !BIAS && !STAGED) {
                const uint16_t *const rbase = o.res + row0 * g.ldr + col0;
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const int r = it * 8 + rr;
                    uint4 v = make_uint4(0, 0, 0, 0);
                    if (r < rows_valid && rc * 8 < cols_valid) {
                        const uint16_t *src = rbase + (uint32_t)(r * ldr + rc * 8);
                        if (rvec && rc * 8 + 8 <= cols_valid) {
                            const v4i t = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(src));   // read once
                            v = make_uint4((uint32_t)t[0], (uint32_t)t[1], (uint32_t)t[2], (uint32_t)t[3]);
                        } else {
                            uint32_t h[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                            for (int j = 0; j < 8; ++j)
                                if (rc * 8 + j < cols_valid) h[j] = src[j];
                            v = make_uint4(h[0] | h[1] << 16, h[2] | h[3] << 16, h[4] | h[5] << 16,
                                           h[6] | h[7] << 16);
                        }
                    }
                    *reinterpret_cast<uint4 *>(region + r * 128 + phys(r, rc) * 16) = v;
                }
            }

            // 2. accumulators -> bf16 in the region (fragment order)
#pragma unroll
            for (int xx = 0; xx < 2; ++xx) {
                const int x = SW ? xx : p * 2 + xx;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int wl = wtile_row0<EPI>(wn, x) + q * 8 + khalf * 4;
                    const v4f sw = BIAS ? *reinterpret_cast<const v4f *>(lds_sw + wl) : sw_r[BIAS ? 0 : x][q];
                    const v4f bias = BIAS ? *reinterpret_cast<const v4f *>(bias_w + (wl - wn * 128)) : v4f{};
                    const v4f swu = SW ? swu_r[x & 1][q] : v4f{};
                    uint2 *dst = reinterpret_cast<uint2 *>(region + l32 * 128 + phys(l32, xx * 4 + q) * 16 + khalf * 8);
                    float v[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int e = q * 4 + j;
                        if (SW) {
                            const float vg = acc[x][y][e] * sa * sw[j];
                            const float vu = acc[x + 2][y][e] * sa * swu[j];
                            v[j] = swiglu_f32(vg, vu);
                        } else {
                            v[j] = acc[x][y][e] * sa * sw[j];
                        }
                    }
                    if (BIAS) {
#pragma unroll
                        for (int j = 0; j < 4; ++j) v[j] += bias[j];
                    } else if (EPI == SPG_EPI_ADD) {
                        const uint2 rv = *dst;
                        v[0] += bf16_lo(rv.x);
                        v[1] += bf16_hi(rv.x);
                        v[2] += bf16_lo(rv.y);
                        v[3] += bf16_hi(rv.y);
                    }
                    *dst = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                }
            }

            // 3. region -> global, 16-byte chunks of whole row segments (all
            // four LDS reads issued before the first store)
            uint4 chunk[4];
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int r = it * 8 + rr;
                chunk[it] = *reinterpret_cast<const uint4 *>(region + r * 128 + phys(r, rc) * 16);
            }
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int r = it * 8 + rr;
                if (r >= rows_valid || rc * 8 >= cols_valid) continue;
                const uint4 v = chunk[it];
                uint16_t *dst = obase + (uint32_t)(r * ldo + rc * 8);
                if (vec16 && rc * 8 + 8 <= cols_valid) {
                    // non-temporal: the output is written once and never read
                    // here, so it should not displace the operand panels from
                    // the caches (measured on 4096 x 34816 x 5120: the main
                    // loop's stage time fell from ~3300 to ~2500 cycles)
                    __builtin_nontemporal_store(v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w}, reinterpret_cast<v4i *>(dst));
                } else {
                    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
                    for (int j = 0; j < 8 && rc * 8 + j < cols_valid; ++j)
                        dst[j] = (uint16_t)(w[j >> 1] >> (16 * (j & 1)));
                }
            }
        }
    }
}

// Fused epilogue of the whole tile (no split).  GIVEN, wave_in: as for
// epilogue_impl.  lds_bias: bias_words<EPI>() floats of LDS, 128 per wave,
// used by nothing else (ADD with a bias row; untouched otherwise).
// STAGE: `region` is this wave's MI * 2 * 4 KiB (one region per pass), and
// whole quadrants of a residual matrix are staged (see STAGED above).
// SO: the output is column segments (g.nseg > 0).  Kernels are instantiated
// apart for it, so the split-output code is not part of the kernels that
// write one output (inside a persistent kernel it cost those 4.5%: more
// scalar spills and twice the code).
template <int EPI, int MI = 4, bool GIVEN = false, bool STAGE = false, bool SO = false>
__device__ __forceinline__ void epilogue(const GemmArgs &g, const Tile &T, const Acc &acc, const float *lds_sa,
                                         const float *lds_sw, float *lds_bias, uint8_t *region, int wave_in = 0)
{
    constexpr bool SW = EPI == SPG_EPI_SWIGLU;
    const int wave = GIVEN ? wave_in : __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int wm = wave >> 1, wn = wave & 1;
    const EpiOut o = epi_out<EPI>(g, T);
    const bool brow = EPI == SPG_EPI_ADD && g.bias_mode != 0;
    if constexpr (SO) {
        // split outputs: one instantiation per bias form, with bounds checks
        if (EPI == SPG_EPI_ADD && brow)
            epilogue_impl<EPI, false, MI, GIVEN, EPI == SPG_EPI_ADD, false, true>(g, T, acc, lds_sa, lds_sw, lds_bias,
                                                                               region, wave_in);
        else
            epilogue_impl<EPI, false, MI, GIVEN, false, false, true>(g, T, acc, lds_sa, lds_sw, lds_bias, region, wave_in);
        return;
    }
    const bool full = T.m0 + wm * (MI * 32) + MI * 32 <= g.M && T.c0 + (SW ? wn * 64 + 64 : wn * 128 + 128) <= o.nvalid &&
                      (((uintptr_t)o.out) & 15) == 0 && (g.ldo & 7) == 0 &&
                      (EPI != SPG_EPI_ADD || brow || ((((uintptr_t)o.res) & 15) == 0 && (g.ldr & 7) == 0));
    if constexpr (EPI == SPG_EPI_ADD) {
        if (brow) {
            if (full)
                epilogue_impl<EPI, true, MI, GIVEN, true>(g, T, acc, lds_sa, lds_sw, lds_bias, region, wave_in);
            else
                epilogue_impl<EPI, false, MI, GIVEN, true>(g, T, acc, lds_sa, lds_sw, lds_bias, region, wave_in);
            return;
        }
        if constexpr (STAGE) {
            // offsets inside the quadrant stay below 2^31 bytes
            if (full && g.ldr < (INT64_C(1) << 23) / MI) {
                epilogue_impl<EPI, true, MI, GIVEN, false, true>(g, T, acc, lds_sa, lds_sw, lds_bias, region, wave_in);
                return;
            }
        }
    }
    if (full)
        epilogue_impl<EPI, true, MI, GIVEN>(g, T, acc, lds_sa, lds_sw, lds_bias, region, wave_in);
    else
        epilogue_impl<EPI, false, MI, GIVEN>(g, T, acc, lds_sa, lds_sw, lds_bias, region, wave_in);
}

}  // namespace gemm
}  // namespace spg
