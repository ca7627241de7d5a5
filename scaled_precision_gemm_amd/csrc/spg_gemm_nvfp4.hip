// NVFP4 block-scaled GEMM for gfx950 (ninfer PR #160, "The NVFP4 TMA route
// reads activation scales as one tile": E2M1 codes with one E4M3 scale per 16
// K-elements, an fp32 tensor scale; linear_add and linear_swiglu at T=4096).
//
//   out = epilogue(t_A t_W * sum_g S^A_g S^W_g sum_{k in g} a_k w_k)
//
// Why not the scaled f8f6f4 MFMA: its block scales are E8M0 (powers of two)
// per 32 K-elements, while NVFP4 scales are E4M3 (4 significant bits) per 16.
// Folding an E4M3 scale into an FP4 or FP8 operand is inexact (code x scale
// needs up to 6 significant bits), and the resulting operand error (2^-4
// relative) would break the GEMM's 2^-12 error budget.  Instead each element
// is decoded once per workgroup tile, on its way into LDS, to the exact f16
// value  e2m1(code) * S * 2^-7  (6 significant bits, range 2^-17 .. 21),
// and the tile is multiplied with v_mfma_f32_32x32x16_f16 (fp32
// accumulation).  The 2^14 of the two operand offsets and the tensor scales
// are applied in the epilogue.  The dense f16 MFMA rate is half the FP8 rate,
// so this path is priced against the f16/bf16 roofline.
//
// Decode without tables: an E2M1 code c placed as f16 bits
// ((c & 7) << 9) | ((c & 8) << 12) is exactly e2m1(c) * 2^-14 (normal codes
// land on exponents 1..3, code 1 on the subnormal 2^-15).  All eight codes of
// a 32-bit word are expanded with byte arithmetic: the high byte of each f16
// is ((c & 7) << 1) | ((c & 8) << 4) and its low byte is zero, so two byte
// permutes (v_perm_b32) assemble four f16 pairs; one packed f16 multiply per
// pair applies S * 2^7 (exact: the product is representable).
#include "spg_gemm_common.h"

namespace spg {

namespace {

using namespace gemm;
constexpr int kBK = 64;   // K elements per stage (32 code bytes, 4 scale bytes per row)

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 decode8_f16(uint32_t w, h2 s2)
{
    const uint32_t lo = w & 0x0F0F0F0Fu;          // codes 0,2,4,6 in bytes 0..3
    const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;   // codes 1,3,5,7
    const uint32_t hl = ((lo << 1) & 0x0E0E0E0Eu) | ((lo << 4) & 0x80808080u);
    const uint32_t hh = ((hi << 1) & 0x0E0E0E0Eu) | ((hi << 4) & 0x80808080u);
    uint32_t d[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        // bytes of dword j: [0, hl.j, 0, hh.j] -> f16 pair (element 2j, 2j+1)
        const uint32_t sel = 0x0Cu | ((uint32_t)j << 8) | (0x0Cu << 16) | ((uint32_t)(4 + j) << 24);
        const uint32_t p = __builtin_amdgcn_perm(hh, hl, sel);
        const h2 v = __builtin_bit_cast(h2, p) * s2;
        d[j] = __builtin_bit_cast(uint32_t, v);
    }
    return make_uint4(d[0], d[1], d[2], d[3]);
}

__device__ __forceinline__ h2 scale_h2(uint32_t code)
{
    const _Float16 h = (_Float16)(decode_e4m3(code) * 128.0f);   // exact: <= 57344, >= 2^-2
    return h2{h, h};
}

template <int EPI>
__global__ __launch_bounds__(kThreads, 1) void gemm_nvfp4_kernel(const GemmArgs g)
{
    constexpr int kLdsBytes = 4 * kStageBytes;
    __shared__ __attribute__((aligned(2048))) uint8_t lds[kLdsBytes];
    // [stage][operand] views of the flat array
    auto lds_ab = [&](int st, int op) -> uint8_t * { return &lds[(st * 2 + op) * kStageBytes]; };
    __shared__ __attribute__((aligned(16))) float lds_sa[kBM];
    __shared__ __attribute__((aligned(16))) float lds_sw[kBN];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const Tile T = tile_of<EPI>(g);

    const int split = blockIdx.y;
    const int64_t k_begin = (int64_t)split * g.k_chunk;
    const int64_t k_end = min(g.K, k_begin + g.k_chunk);
    const int nk = (int)((k_end - k_begin + kBK - 1) / kBK);

    stage_scales<EPI, SPG_FMT_NVFP4>(g, T, lds_sa, lds_sw);

    // ---- this thread stages row tid of the A tile and row tid of the W tile
    const int64_t G = g.K / 16;
    const bool aok = T.m0 + tid < g.M;
    bool wok;
    const int64_t wr = w_row<EPI>(g, T, tid, wok);
    const uint8_t *acode = g.A + (aok ? T.m0 + tid : 0) * g.lda;
    const uint8_t *wcode = g.W + (wok ? wr : 0) * g.ldw;
    const uint8_t *ascl = (const uint8_t *)g.sa + (aok ? T.m0 + tid : 0) * G;
    const uint8_t *wscl = (const uint8_t *)g.sw + (wok ? wr : 0) * G;

    uint4 ca[2], cw[2];
    uint32_t sa4, sw4;
    auto gload = [&](int64_t k0) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const bool kin = k0 + 32 * h < k_end;
            ca[h] = (aok && kin) ? *reinterpret_cast<const uint4 *>(acode + k0 / 2 + 16 * h) : make_uint4(0, 0, 0, 0);
            cw[h] = (wok && kin) ? *reinterpret_cast<const uint4 *>(wcode + k0 / 2 + 16 * h) : make_uint4(0, 0, 0, 0);
        }
        sa4 = 0;
        sw4 = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (k0 + 16 * q < k_end) {
                if (aok) sa4 |= (uint32_t)ascl[k0 / 16 + q] << (8 * q);
                if (wok) sw4 |= (uint32_t)wscl[k0 / 16 + q] << (8 * q);
            }
        }
    };
    auto swrite = [&](int st) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const uint4 &va = ca[c >> 2];
            const uint4 &vw = cw[c >> 2];
            const uint32_t wa = (c & 3) == 0 ? va.x : (c & 3) == 1 ? va.y : (c & 3) == 2 ? va.z : va.w;
            const uint32_t ww = (c & 3) == 0 ? vw.x : (c & 3) == 1 ? vw.y : (c & 3) == 2 ? vw.z : vw.w;
            const int q = c >> 1;
            *reinterpret_cast<uint4 *>(lds_ab(st, 0) + swz(tid, c)) = decode8_f16(wa, scale_h2((sa4 >> (8 * q)) & 0xFFu));
            *reinterpret_cast<uint4 *>(lds_ab(st, 1) + swz(tid, c)) = decode8_f16(ww, scale_h2((sw4 >> (8 * q)) & 0xFFu));
        }
    };

    Acc acc;
    zero_acc(acc);
    const int l32 = lane & 31, khalf = lane >> 5;
    auto brow = [&](int ni) -> uint32_t { return (uint32_t)wtile_row0<EPI>(wn, ni) + l32; };
    auto compute = [&](int st) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            // 8 f16 of K per lane: lanes 0..31 chunk 2 ks, lanes 32..63 chunk 2 ks + 1
            const uint32_t c = ks * 2 + khalf;
            v8h af[4], bf[4];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
                af[mi] = __builtin_bit_cast(v8h, *reinterpret_cast<const uint4 *>(lds_ab(st, 0) + swz(wm * 128 + mi * 32 + l32, c)));
#pragma unroll
            for (int ni = 0; ni < 4; ++ni)
                bf[ni] = __builtin_bit_cast(v8h, *reinterpret_cast<const uint4 *>(lds_ab(st, 1) + swz(brow(ni), c)));
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < 4; ++ni)
                    acc[ni][mi] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[ni], af[mi], acc[ni][mi], 0, 0, 0);
        }
    };

    if (nk > 0) {
        gload(k_begin);
        swrite(0);
    }
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const bool more = kt + 1 < nk;
        if (more) gload(k_begin + (int64_t)(kt + 1) * kBK);
        compute(kt & 1);
        if (more) swrite((kt + 1) & 1);
        __syncthreads();
    }

    if (g.split_k > 1) {
        splitk_store(g, T, acc);      // the slices are summed by splitk_reduce_kernel
        return;
    }
    epilogue<EPI>(g, T, acc, lds_sa, lds_sw, &lds[(threadIdx.x >> 6) * 4096]);   // after the barrier above
}

template <int EPI>
hipError_t launch_epi(const GemmArgs &g, const spg_plan &p, hipStream_t s)
{
    dim3 grid((unsigned)p.tiles, (unsigned)g.split_k, 1);
    gemm_nvfp4_kernel<EPI><<<grid, kThreads, 0, s>>>(g);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && g.split_k > 1) e = launch_splitk_reduce(g, p.tiles, s);
    return e;
}

}  // namespace

hipError_t launch_gemm_nvfp4(const GemmArgs &g, const spg_plan &p, hipStream_t s)
{
    switch (g.epilogue) {
    case SPG_EPI_STORE: return launch_epi<SPG_EPI_STORE>(g, p, s);
    case SPG_EPI_ADD: return launch_epi<SPG_EPI_ADD>(g, p, s);
    default: return launch_epi<SPG_EPI_SWIGLU>(g, p, s);
    }
}

}  // namespace spg
