// Split-K, part 2: sum the fp32 partial tiles of the K slices and apply the
// fused epilogue.  Runs after the GEMM kernel on the same stream, so every
// slice's stores are complete and visible.  One workgroup per (tile, 32x32
// accumulator block) - 16 per tile, 8 for SWIGLU, whose workgroups take a
// gate block and its up block - so the reduction of a tile is spread over
// many compute units; each thread sums its 16 accumulators over the slices
// in slice order (deterministic) and applies the same epilogue code as the
// unsplit kernel.
#include "spg_gemm_common.h"

namespace spg {

namespace {

using namespace gemm;

template <int EPI, int SMODE>
__global__ __launch_bounds__(kThreads) void splitk_reduce_kernel(const GemmArgs g)
{
    __shared__ __attribute__((aligned(16))) float lds_sa[kBM];
    __shared__ __attribute__((aligned(16))) float lds_sw[kBN];
    const Tile T = tile_from_id<EPI>(g, g.tile_begin + blockIdx.x);
    // the tile's scale factors: loads issued now, written to LDS once the
    // partial sums are in (a wait for them before the partial loads are
    // issued would serialize the two)
    float va, vw;
    scale_values<EPI, SMODE>(g, T, va, vw);

    // Thread i handles the 16 accumulators thread i of the GEMM workgroup
    // held for block (x, y), so the GEMM's epilogue code applies unchanged.
    const int x = (int)blockIdx.y >> 2;    // SWIGLU: 0..1 (gate blocks), else 0..3
    const int y = (int)blockIdx.y & 3;
    // the layout splitk_store writes: element 4q + r of block b of thread i
    // at (4b + q) * 1024 + 4i + r within a (tile, slice) partial
    const float *tile_base = g.partials + (int64_t)blockIdx.x * g.split_k * (kBM * kBN) + threadIdx.x * 4;
    // The slices of a block (and of its up partner for SWIGLU) are loaded
    // four at a time, every load issued before any is summed, then added in
    // slice order (deterministic; the same order as one slice at a time).
    auto load_part = [&](int s, int blk, v4f (&p)[4]) {
        const float *src = tile_base + (int64_t)s * (kBM * kBN) + blk * 4 * (kThreads * 4);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            p[q] = __builtin_nontemporal_load(reinterpret_cast<const v4f *>(src + q * (kThreads * 4)));
    };
    auto add_part = [&](int s, const v4f (&p)[4], v16f &t) {
        v16f v;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            v[4 * q] = p[q][0];
            v[4 * q + 1] = p[q][1];
            v[4 * q + 2] = p[q][2];
            v[4 * q + 3] = p[q][3];
        }
        t = s == 0 ? v : t + v;
    };
    constexpr bool SW = EPI == SPG_EPI_SWIGLU;
    // only token rows below M were stored (the others are not read, and the
    // epilogue skips them)
    const bool live = T.m0 + (int64_t)(threadIdx.x >> 7) * 128 + y * 32 + (threadIdx.x & 31) < g.M;
    v16f acc = {}, acc_up = {};
    if (live) {
        for (int s0 = 0; s0 < g.split_k; s0 += 4) {
            v4f p[4][4], pu[4][4];
#pragma unroll
            for (int d = 0; d < 4; ++d)
                if (s0 + d < g.split_k) {
                    load_part(s0 + d, x * 4 + y, p[d]);
                    if (SW) load_part(s0 + d, (x + 2) * 4 + y, pu[d]);
                }
#pragma unroll
            for (int d = 0; d < 4; ++d)
                if (s0 + d < g.split_k) {
                    add_part(s0 + d, p[d], acc);
                    if (SW) add_part(s0 + d, pu[d], acc_up);
                }
        }
    }
    lds_sa[threadIdx.x] = va;
    lds_sw[threadIdx.x] = vw;
    __syncthreads();   // scales staged

    const int wn = (threadIdx.x >> 6) & 1;
    epilogue_block<EPI>(g, T, epi_out<EPI>(g, T), wtile_row0<EPI>(wn, x), y, acc, EPI == SPG_EPI_SWIGLU ? acc_up : acc,
                        lds_sa, lds_sw);
}

template <int EPI>
hipError_t launch_epi(const GemmArgs &g, int64_t tiles, hipStream_t s)
{
    const dim3 grid((unsigned)tiles, EPI == SPG_EPI_SWIGLU ? 8u : 16u);
    if (g.format == SPG_FMT_E4M3_ROW)
        splitk_reduce_kernel<EPI, SPG_FMT_E4M3_ROW><<<grid, kThreads, 0, s>>>(g);
    else if (g.format == SPG_FMT_E4M3_TENSOR)
        splitk_reduce_kernel<EPI, SPG_FMT_E4M3_TENSOR><<<grid, kThreads, 0, s>>>(g);
    else
        splitk_reduce_kernel<EPI, SPG_FMT_NVFP4><<<grid, kThreads, 0, s>>>(g);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_splitk_reduce(const GemmArgs &g, int64_t tiles, hipStream_t s)
{
    switch (g.epilogue) {
    case SPG_EPI_STORE: return launch_epi<SPG_EPI_STORE>(g, tiles, s);
    case SPG_EPI_ADD: return launch_epi<SPG_EPI_ADD>(g, tiles, s);
    default: return launch_epi<SPG_EPI_SWIGLU>(g, tiles, s);
    }
}

}  // namespace spg
