// FP8 E4M3 scaled GEMM for gfx950 with fused bf16 epilogues.
//
// out = epilogue(s_a * s_w * sum_k a_k w_k), A [M,K] and W [N,K] K-contiguous
// (the NT layout of AstrAI's "E4M3, NT pre-quantized" benchmark), fp32
// accumulation with the scales applied after it, as ninfer PR #167 states for
// its row-scaled A8 GEMM (opening summary: same accumulator, scale
// application, epilogue and output policies for the linear, linear_add and
// linear_swiglu call sites).
//
// Design for CDNA4 (the pages' sm_120 / L20 kernels are prior art only):
//  * workgroup tile 256 x 256 outputs, 4 waves in a 2 x 2 arrangement, each
//    wave owning a 128 x 128 sub-tile = 4 x 4 blocks of
//    v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3 -> fp32).  Operand reuse per
//    LDS read is what PR #167's wider warp tile buys (its table: MMA per
//    operand load 8 -> 32); here each 32-byte A fragment and each B fragment
//    feeds 4 MFMAs of 131072 flops.
//  * K advances 128 bytes per stage.  Each thread loads 8 + 8 sixteen-byte
//    vectors per stage (a wave covers 8 whole 128-byte row segments), keeps
//    them in registers while the MFMAs of the current stage run, then writes
//    them into the other of two LDS buffers; one barrier per stage.
//  * LDS rows are 128 bytes with the XOR chunk swizzle of spg_gemm_common.h.
//  * SWIGLU pairs weight rows inside one 256-row W tile (128 gate + 128 up).
//  * XCD-aware tile order, optional split-K through the workspace.
#include "spg_gemm_common.h"

namespace spg {

namespace {

using namespace gemm;
constexpr int kBK = 128;   // K bytes (= E4M3 elements) per stage

template <int EPI, int SMODE>
__global__ __launch_bounds__(kThreads, 1) void gemm_fp8_kernel(const GemmArgs g)
{
    __shared__ __attribute__((aligned(1024))) uint8_t lds_ab[2][2][kStageBytes];
    __shared__ float lds_sa[kBM];
    __shared__ float lds_sw[kBN];
    __shared__ uint32_t lds_flag;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const Tile T = tile_of<EPI>(g);

    const uint8_t *A = g.A + (g.stride_a ? T.b * g.stride_a : 0);
    const uint8_t *W = g.W + (g.stride_w ? T.b * g.stride_w : 0);

    const int split = blockIdx.y;
    const int64_t k_begin = (int64_t)split * g.k_chunk;
    const int64_t k_end = min(g.K, k_begin + g.k_chunk);
    const int nk = (int)((k_end - k_begin + kBK - 1) / kBK);

    // ---- scales into LDS (read by the epilogue after the main loop) ---------
    {
        bool wok;
        const int64_t wr = w_row<EPI>(g, T, tid, wok);
        const int64_t r = T.m0 + tid;
        if (SMODE == SPG_FMT_E4M3_ROW) {
            const float *sa = (const float *)g.sa + (g.stride_a ? T.b * g.sa_bstride : 0);
            const float *sw = (const float *)g.sw + (g.stride_w ? T.b * g.sw_bstride : 0);
            lds_sa[tid] = r < g.M ? sa[r] : 0.0f;
            lds_sw[tid] = wok ? sw[wr] : 0.0f;
        } else {
            lds_sa[tid] = ((const float *)g.sa)[g.stride_a ? T.b : 0];
            lds_sw[tid] = ((const float *)g.sw)[g.stride_w ? T.b : 0];
        }
    }

    // ---- global -> register loads -------------------------------------------
    // Thread tid moves 16-byte chunk (tid & 7) of tile rows (tid >> 3) + 32 i,
    // i = 0..7, for A and for W.  Rows i sit at uniform offsets of 32 i rows
    // from the thread's first row (W: separate bases for rows 0..127 and
    // 128..255, which SWIGLU maps to the gate and up halves).
    const int crow = tid >> 3, cc = tid & 7;
    bool ok0, ok4;
    const int64_t wr0 = w_row<EPI>(g, T, crow, ok0);
    const int64_t wr4 = w_row<EPI>(g, T, crow + 128, ok4);
    const uint8_t *abase = A + (T.m0 + crow) * g.lda;
    const uint8_t *wbase0 = W + wr0 * g.ldw;
    const uint8_t *wbase1 = W + wr4 * g.ldw;
    uint32_t aok = 0, wok = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (T.m0 + crow + 32 * i < g.M) aok |= 1u << i;
        bool ok;
        (void)w_row<EPI>(g, T, crow + 32 * i, ok);
        if (ok) wok |= 1u << i;
    }
    uint4 ra[8], rw[8];
    auto gload = [&](int64_t k0) {
        const int64_t kk = k0 + cc * 16;
        const bool kin = kk < k_end;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint8_t *ap = abase + (int64_t)(32 * i) * g.lda + kk;
            const uint8_t *wp = (i < 4 ? wbase0 : wbase1) + (int64_t)(32 * (i & 3)) * g.ldw + kk;
            ra[i] = (kin && (aok >> i & 1)) ? *reinterpret_cast<const uint4 *>(ap) : make_uint4(0, 0, 0, 0);
            rw[i] = (kin && (wok >> i & 1)) ? *reinterpret_cast<const uint4 *>(wp) : make_uint4(0, 0, 0, 0);
        }
    };
    auto swrite = [&](int st) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t r = crow + 32 * i;
            *reinterpret_cast<uint4 *>(&lds_ab[st][0][swz(r, cc)]) = ra[i];
            *reinterpret_cast<uint4 *>(&lds_ab[st][1][swz(r, cc)]) = rw[i];
        }
    };

    // ---- MFMA main loop -------------------------------------------------------
    Acc acc;
    zero_acc(acc);
    const int l32 = lane & 31, khalf = lane >> 5;
    // LDS W-tile row of lane l32 in column block ni: SWIGLU blocks 0,1 are gate
    // rows and blocks 2,3 the up rows of the same output columns.
    auto brow = [&](int ni) -> uint32_t {
        if (EPI == SPG_EPI_SWIGLU) return (ni < 2 ? wn * 64 + ni * 32 : 128 + wn * 64 + (ni - 2) * 32) + l32;
        return wn * 128 + ni * 32 + l32;
    };
    auto frag = [&](const uint8_t *base, uint32_t r, uint32_t c) -> v8i {
        const uint4 lo = *reinterpret_cast<const uint4 *>(base + swz(r, c));
        const uint4 hi = *reinterpret_cast<const uint4 *>(base + swz(r, c + 1));
        return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };
    auto compute = [&](int st) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            // 32 bytes of K per lane: lanes 0..31 take chunks c0, c0+1 of the
            // 64-byte K step, lanes 32..63 the next two chunks.  A and B use
            // the same K placement, so any per-instruction K order of the
            // hardware sums the same products.
            const uint32_t c0 = ks * 4 + khalf * 2;
            v8i af[4], bf[4];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) af[mi] = frag(lds_ab[st][0], wm * 128 + mi * 32 + l32, c0);
#pragma unroll
            for (int ni = 0; ni < 4; ++ni) bf[ni] = frag(lds_ab[st][1], brow(ni), c0);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi)
#pragma unroll
                for (int ni = 0; ni < 4; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[mi], bf[ni], acc[mi][ni],
                                                                                  0, 0, 0, 0, 0, 0);
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

    if (g.split_k > 1 && !splitk_fixup(g, T, acc, &lds_flag)) return;
    epilogue<EPI>(g, T, acc, lds_sa, lds_sw);
}

__global__ void zero_u32_kernel(uint32_t *p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

template <int EPI>
hipError_t launch_epi(const GemmArgs &g, const spg_plan &p, hipStream_t s)
{
    if (g.split_k > 1) {
        zero_u32_kernel<<<dim3((unsigned)((p.tiles + 255) / 256)), 256, 0, s>>>(g.counters, p.tiles);
    }
    dim3 grid((unsigned)p.tiles, (unsigned)g.split_k, 1);
    if (g.format == SPG_FMT_E4M3_ROW)
        gemm_fp8_kernel<EPI, SPG_FMT_E4M3_ROW><<<grid, kThreads, 0, s>>>(g);
    else
        gemm_fp8_kernel<EPI, SPG_FMT_E4M3_TENSOR><<<grid, kThreads, 0, s>>>(g);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_fp8(const GemmArgs &g, const spg_plan &p, hipStream_t s)
{
    switch (g.epilogue) {
    case SPG_EPI_STORE: return launch_epi<SPG_EPI_STORE>(g, p, s);
    case SPG_EPI_ADD: return launch_epi<SPG_EPI_ADD>(g, p, s);
    default: return launch_epi<SPG_EPI_SWIGLU>(g, p, s);
    }
}

}  // namespace spg
