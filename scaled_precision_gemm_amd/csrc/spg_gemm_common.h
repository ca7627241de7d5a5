// Pieces shared by the FP8 and NVFP4 GEMM kernels: tile scheduling, the LDS
// layout of a K stage, split-K fixup and the fused bf16 epilogues.
//
// Both kernels use a 256 x 256 workgroup tile computed by 4 waves (2 x 2),
// each wave a 128 x 128 sub-tile of 4 x 4 32x32 MFMA blocks.  The 32x32 MFMA
// accumulator layout is the same for every input format: lane l, register e
// of a block holds row (e / 4) * 8 + (l / 32) * 4 + (e % 4), column l % 32.
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

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + __expf(-z)); }

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
template <int EPI>
__device__ __forceinline__ Tile tile_from_id(const GemmArgs &g, int64_t t)
{
    Tile T;
    T.global = t;
    const int64_t per = g.tiles_m * g.tiles_n;
    T.b = t / per;
    t -= T.b * per;
    const int64_t span = (int64_t)kGroupM * g.tiles_n;
    const int64_t first_m = (t / span) * kGroupM;
    const int64_t gm = min((int64_t)kGroupM, g.tiles_m - first_m);
    const int64_t tin = t % span;
    T.m0 = (first_m + tin % gm) * kBM;
    T.tn = tin / gm;
    T.n0 = EPI == SPG_EPI_SWIGLU ? T.tn * (kBN / 2) : T.tn * kBN;
    T.c0 = T.n0;
    return T;
}

template <int EPI>
__device__ __forceinline__ Tile tile_of(const GemmArgs &g)
{
    return tile_from_id<EPI>(g, xcd_remap(blockIdx.x, gridDim.x));
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

using Acc = v16f[4][4];

__device__ __forceinline__ void zero_acc(Acc &acc)
{
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[mi][ni][e] = 0.0f;
}

// Split-K, part 1: every K slice stores its fp32 partial tile and stops; a
// second kernel (splitk_reduce_kernel) sums the slices once all have
// finished - the kernel boundary orders the stores before the loads, so no
// device-scope fence or counter is needed.  A lane's 16 accumulators of one
// 32x32 block are stored contiguously (four 16-byte stores; a wave writes
// 4 KiB contiguous per block): slice s of tile t, block b, thread x starts at
// ((t * S + s) * 16 + b) * 4096 + x * 16 floats.
__device__ __forceinline__ void splitk_store(const GemmArgs &g, const Tile &T, const Acc &acc)
{
    float *base = g.partials + (T.global * g.split_k + blockIdx.y) * (int64_t)(kBM * kBN) + threadIdx.x * 16;
#pragma unroll
    for (int blk = 0; blk < 16; ++blk) {
        v4f *dst = reinterpret_cast<v4f *>(base + blk * (kThreads * 16));
        const v16f &a = acc[blk >> 2][blk & 3];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            __builtin_nontemporal_store(v4f{a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]}, dst + q);
    }
}

// LDS-staged fused epilogue.
//  1. (ADD) the residual tile is copied into LDS with coalesced loads;
//  2. every lane forms its outputs from the accumulators:
//       v = acc * lds_sa[row] * lds_sw[col]   (per-row / per-tensor FP8 scales,
//           or the NVFP4 tensor-scale product in lds_sa with lds_sw = 1)
//       STORE: bf16(v); ADD: bf16(v + residual) with the residual read back
//       from LDS in fp32 (one rounding); SWIGLU: bf16(silu(gate) * up) with
//       gate in column blocks 0,1 and up in blocks 2,3 of the same lanes
//     and writes the bf16 result into a row-major LDS tile;
//  3. the tile leaves LDS as 16-byte row segments (one wave stores two whole
//     512-byte rows per instruction), falling back to 2-byte stores for
//     unaligned outputs and for the ragged right edge.
// AstrAI's commit log describes the same idea on its hardware (stage the
// epilogue through shared memory, then coalesced 16-byte copy-out).
// `tile` must hold kEpiRows * kEpiStride bytes and be free of other use.
constexpr int kEpiStride = 528;                // bytes per LDS row: 512 + 16 pad
constexpr int kEpiBytes = kBM * kEpiStride;    // 135168

template <int EPI>
__device__ __forceinline__ void epilogue(const GemmArgs &g, const Tile &T, const Acc &acc,
                                         const float *lds_sa, const float *lds_sw, uint8_t *tile)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, khalf = lane >> 5;
    uint16_t *out = (uint16_t *)g.out + (g.stride_o ? T.b * g.stride_o : 0);
    const uint16_t *res = g.residual ? g.residual + (g.stride_r ? T.b * g.stride_r : 0) : nullptr;
    const int64_t nvalid = EPI == SPG_EPI_SWIGLU ? g.N / 2 : g.N;
    constexpr int NCOL = EPI == SPG_EPI_SWIGLU ? kBN / 2 : kBN;   // output columns of the tile
    constexpr int CPR = NCOL / 8;                                 // 16-byte chunks per row
    const int64_t rows_valid = min((int64_t)kBM, g.M - T.m0);
    const int64_t cols_valid = min((int64_t)NCOL, nvalid - T.c0);

    // 1. residual tile -> LDS
    if (EPI == SPG_EPI_ADD) {
        const bool vec = ((((uintptr_t)res) & 15) == 0) && ((g.ldr & 7) == 0);
        for (int q = tid; q < kBM * CPR; q += kThreads) {
            const int r = q / CPR, c = (q % CPR) * 8;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (r < rows_valid) {
                const uint16_t *src = res + (T.m0 + r) * g.ldr + T.c0 + c;
                if (vec && c + 8 <= cols_valid) {
                    v = *reinterpret_cast<const uint4 *>(src);
                } else {
                    uint16_t h[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                    for (int j = 0; j < 8; ++j)
                        if (c + j < cols_valid) h[j] = src[j];
                    v = make_uint4(h[0] | (uint32_t)h[1] << 16, h[2] | (uint32_t)h[3] << 16,
                                   h[4] | (uint32_t)h[5] << 16, h[6] | (uint32_t)h[7] << 16);
                }
            }
            *reinterpret_cast<uint4 *>(tile + r * kEpiStride + c * 2) = v;
        }
        __syncthreads();
    }

    // 2. accumulators -> bf16 tile in LDS
    constexpr int NB = EPI == SPG_EPI_SWIGLU ? 2 : 4;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int ni = 0; ni < NB; ++ni) {
            const int cl = EPI == SPG_EPI_SWIGLU ? wn * 64 + ni * 32 + l32 : wn * 128 + ni * 32 + l32;
            const float swc = lds_sw[cl];
            const float swu = EPI == SPG_EPI_SWIGLU ? lds_sw[128 + cl] : 0.0f;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int rl = wm * 128 + mi * 32 + (e >> 2) * 8 + khalf * 4 + (e & 3);
                uint16_t *dst = reinterpret_cast<uint16_t *>(tile + rl * kEpiStride) + cl;
                const float sa = lds_sa[rl];
                float v;
                if (EPI == SPG_EPI_SWIGLU) {
                    const float vg = acc[mi][ni][e] * sa * swc;
                    const float vu = acc[mi][ni + 2][e] * sa * swu;
                    v = silu_f32(vg) * vu;
                } else {
                    v = acc[mi][ni][e] * sa * swc;
                    if (EPI == SPG_EPI_ADD) v += bf16_lo(*dst);
                }
                *dst = (uint16_t)f32_to_bf16(v);
            }
        }
    }
    __syncthreads();

    // 3. LDS -> global, 16-byte row segments
    const bool vec = ((((uintptr_t)out) & 15) == 0) && ((g.ldo & 7) == 0);
    for (int q = tid; q < kBM * CPR; q += kThreads) {
        const int r = q / CPR, c = (q % CPR) * 8;
        if (r >= rows_valid || c >= cols_valid) continue;
        const uint4 v = *reinterpret_cast<const uint4 *>(tile + r * kEpiStride + c * 2);
        uint16_t *dst = out + (T.m0 + r) * g.ldo + T.c0 + c;
        if (vec && c + 8 <= cols_valid) {
            *reinterpret_cast<uint4 *>(dst) = v;
        } else {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
            for (int j = 0; j < 8 && c + j < cols_valid; ++j) dst[j] = (uint16_t)(w[j >> 1] >> (16 * (j & 1)));
        }
    }
}

}  // namespace gemm
}  // namespace spg
