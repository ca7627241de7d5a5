// Split-K, part 2: sum the fp32 partial tiles of the K slices and apply the
// fused epilogue.  Runs after the GEMM kernel on the same stream, so every
// slice's stores are complete and visible.  One workgroup per (tile, 32x32
// accumulator block) - 16 per tile, 8 for SWIGLU, whose workgroups take a
// gate block and its up block - so the reduction of a tile is spread over
// many compute units; each thread sums its 16 accumulators over the slices
// in slice order (deterministic) with all 16-byte loads in flight.
#include "spg_gemm_common.h"

namespace spg {

namespace {

using namespace gemm;

template <int EPI, int SMODE>
__global__ __launch_bounds__(kThreads) void splitk_reduce_kernel(const GemmArgs g)
{
    const Tile T = tile_from_id<EPI>(g, blockIdx.x);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, khalf = lane >> 5;
    const int mi = EPI == SPG_EPI_SWIGLU ? (int)blockIdx.y >> 1 : (int)blockIdx.y >> 2;
    const int ni = EPI == SPG_EPI_SWIGLU ? (int)blockIdx.y & 1 : (int)blockIdx.y & 3;

    const float *tile_base = g.partials + T.global * g.split_k * (int64_t)(kBM * kBN) + tid * 16;
    auto sum_block = [&](int blk) -> v16f {
        v16f t;
        for (int s = 0; s < g.split_k; ++s) {
            const v4f *src = reinterpret_cast<const v4f *>(tile_base + ((int64_t)s * 16 + blk) * (kThreads * 16));
            v16f p;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const v4f v = __builtin_nontemporal_load(src + q);
                p[4 * q] = v[0];
                p[4 * q + 1] = v[1];
                p[4 * q + 2] = v[2];
                p[4 * q + 3] = v[3];
            }
            t = s == 0 ? p : t + p;
        }
        return t;
    };
    const v16f acc = sum_block(mi * 4 + ni);
    const v16f acc_up = EPI == SPG_EPI_SWIGLU ? sum_block(mi * 4 + ni + 2) : v16f{};

    const int cl = EPI == SPG_EPI_SWIGLU ? wn * 64 + ni * 32 + l32 : wn * 128 + ni * 32 + l32;
    const int64_t nvalid = EPI == SPG_EPI_SWIGLU ? g.N / 2 : g.N;
    const int64_t col = T.c0 + cl;
    if (col >= nvalid) return;

    // scales, applied in the main epilogue's order (acc * sa * sw): per-row or
    // per-tensor FP8, or the NVFP4 tensor-scale product with sw = 1
    float swc = 1.0f, swu = 1.0f, s_tensor = 1.0f;
    const float *sa = nullptr;
    if (SMODE == SPG_FMT_E4M3_ROW) {
        sa = (const float *)g.sa + (g.stride_a ? T.b * g.sa_bstride : 0);
        const float *sw = (const float *)g.sw + (g.stride_w ? T.b * g.sw_bstride : 0);
        swc = sw[T.n0 + cl];
        if (EPI == SPG_EPI_SWIGLU) swu = sw[g.N / 2 + T.n0 + cl];
    } else if (SMODE == SPG_FMT_E4M3_TENSOR) {
        s_tensor = ((const float *)g.sa)[g.stride_a ? T.b : 0];
        swc = ((const float *)g.sw)[g.stride_w ? T.b : 0];
    } else {
        s_tensor = 16384.0f * *g.tscale_a * *g.tscale_w;
    }

    uint16_t *out = (uint16_t *)g.out + (g.stride_o ? T.b * g.stride_o : 0);
    const uint16_t *res = g.residual ? g.residual + (g.stride_r ? T.b * g.stride_r : 0) : nullptr;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int64_t row = T.m0 + wm * 128 + mi * 32 + (e >> 2) * 8 + khalf * 4 + (e & 3);
        if (row >= g.M) continue;
        const float sr = SMODE == SPG_FMT_E4M3_ROW ? sa[row] : s_tensor;
        float v;
        if (EPI == SPG_EPI_SWIGLU) {
            const float vg = acc[e] * sr * swc;
            const float vu = acc_up[e] * sr * swu;
            v = silu_f32(vg) * vu;
        } else {
            v = acc[e] * sr * swc;
            if (EPI == SPG_EPI_ADD) v += bf16_lo(res[row * g.ldr + col]);
        }
        out[row * g.ldo + col] = (uint16_t)f32_to_bf16(v);
    }
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
