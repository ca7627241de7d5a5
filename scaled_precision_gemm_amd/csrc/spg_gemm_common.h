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

// Byte offset of 16-byte chunk `chunk` (0..7) of LDS row `row`.  The XOR with
// row & 7 spreads the same logical chunk of eight consecutive rows over all
// eight 16-byte bank groups of a 128-byte row.  Stage buffers are aligned to
// the 1 KiB period of this pattern.
__device__ __forceinline__ uint32_t swz(uint32_t row, uint32_t chunk)
{
    return row * kRowBytes + ((chunk ^ (row & 7u)) << 4);
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
__device__ __forceinline__ Tile tile_of(const GemmArgs &g)
{
    Tile T;
    int64_t t = xcd_remap(blockIdx.x, gridDim.x);
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

// Split-K: every K slice stores its fp32 partial tile (register order, so
// each store instruction writes 1 KiB contiguous per wave); the slice that
// arrives last (device-scope counter, zeroed before the launch) sums all
// partials in slice order and goes on to the epilogue.  Returns false for
// the slices that stop here.
__device__ __forceinline__ bool splitk_fixup(const GemmArgs &g, const Tile &T, Acc &acc, uint32_t *flag)
{
    const int tid = threadIdx.x;
    const int split = blockIdx.y;
    constexpr int64_t kTileElems = (int64_t)kBM * kBN;
    float *mine = g.partials + (T.global * g.split_k + split) * kTileElems;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e) mine[((mi * 4 + ni) * 16 + e) * kThreads + tid] = acc[mi][ni][e];
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = atomicAdd(&g.counters[T.global], 1u);
        *flag = (prev == (uint32_t)g.split_k - 1) ? 1u : 0u;
    }
    __syncthreads();
    if (!*flag) return false;
    __threadfence();
    const float *all = g.partials + T.global * g.split_k * kTileElems;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                float s = 0.0f;
                for (int sp = 0; sp < g.split_k; ++sp)
                    s += __builtin_nontemporal_load(&all[sp * kTileElems + ((mi * 4 + ni) * 16 + e) * kThreads + tid]);
                acc[mi][ni][e] = s;
            }
    return true;
}

// Fused epilogue.  v = acc * lds_sa[row] * lds_sw[col] (per-row/per-tensor
// FP8 scales, or the NVFP4 tensor-scale product in lds_sa with lds_sw = 1),
// then STORE / ADD (fp32 residual add before the single bf16 rounding) /
// SWIGLU (silu(gate) * up with gate in blocks 0,1 and up in blocks 2,3 of
// the same lanes).
template <int EPI>
__device__ __forceinline__ void epilogue(const GemmArgs &g, const Tile &T, const Acc &acc,
                                         const float *lds_sa, const float *lds_sw)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, khalf = lane >> 5;
    uint16_t *out = (uint16_t *)g.out + (g.stride_o ? T.b * g.stride_o : 0);
    const uint16_t *res = g.residual ? g.residual + (g.stride_r ? T.b * g.stride_r : 0) : nullptr;
    const int64_t nvalid = EPI == SPG_EPI_SWIGLU ? g.N / 2 : g.N;
    constexpr int NB = EPI == SPG_EPI_SWIGLU ? 2 : 4;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
        for (int ni = 0; ni < NB; ++ni) {
            const int cl = EPI == SPG_EPI_SWIGLU ? wn * 64 + ni * 32 + l32 : wn * 128 + ni * 32 + l32;
            const int64_t col = T.c0 + cl;
            if (col >= nvalid) continue;
            const float swc = lds_sw[cl];
            const float swu = EPI == SPG_EPI_SWIGLU ? lds_sw[128 + cl] : 0.0f;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int rl = wm * 128 + mi * 32 + (e >> 2) * 8 + khalf * 4 + (e & 3);
                const int64_t row = T.m0 + rl;
                if (row >= g.M) continue;
                const float sa = lds_sa[rl];
                float v;
                if (EPI == SPG_EPI_SWIGLU) {
                    const float vg = acc[mi][ni][e] * sa * swc;
                    const float vu = acc[mi][ni + 2][e] * sa * swu;
                    v = silu_f32(vg) * vu;
                } else {
                    v = acc[mi][ni][e] * sa * swc;
                    if (EPI == SPG_EPI_ADD) v += bf16_lo(res[row * g.ldr + col]);
                }
                out[row * g.ldo + col] = (uint16_t)f32_to_bf16(v);
            }
        }
    }
}

}  // namespace gemm
}  // namespace spg
