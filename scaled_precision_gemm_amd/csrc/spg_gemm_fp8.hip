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
//  * Workgroup tile 256 x 256 outputs, 4 waves (2 x 2), each wave a 128 x 128
//    sub-tile = 4 x 4 blocks of v_mfma_f32_32x32x64_f8f6f4 (E4M3 x E4M3 ->
//    fp32; 256 accumulators per lane).  Each 32-byte A or B fragment read
//    from LDS feeds 4 MFMAs of 131072 flops (PR #167's table makes the same
//    point about operand reuse per load on its hardware).
//  * K advances 128 bytes per stage, two LDS slots of 64 KiB.  Global data
//    moves straight into LDS with buffer_load_dwordx4 ... lds (no register
//    staging); eight lanes cover one whole 128-byte row segment, the unit the
//    memory path moves efficiently (measured: 24.7 TB/s into LDS chip-wide
//    with 128-byte segments, 14.2 with 64-byte ones).  Out-of-range rows and
//    the K tail read as zero through the buffer range check.
//  * LDS rows are 128 bytes; chunk c of row r sits at chunk c ^ ((r >> 1) & 7)
//    (spg_gemm_common.h), applied on the global side of the copy: each lane
//    fetches the chunk that belongs in its fixed LDS slot.
//  * A stage is two K=64 sub-steps with two fragment register sets.  Two
//    barriers per stage: after the stage's second fragment set is in
//    registers ("slot free": the copy of stage kt+2 starts), and before the
//    last 4 MFMAs ("stage kt+1 published": its first fragments are read while
//    those MFMAs run).  A copy thus has about 1.4 stages to land.
//  * SWIGLU pairs weight rows inside one 256-row W tile (128 gate + 128 up).
//  * XCD-aware tile order; optional split-K through the workspace;
//    epilogue straight from registers with 8-byte stores (W fragments are the
//    first MFMA operand, so a lane holds four adjacent output columns).
#include "spg_gemm_common.h"

namespace spg {

namespace {

using namespace gemm;
constexpr int kBK = 128;                      // K bytes (E4M3 elements) per stage
constexpr int kOp = kBM * kBK;                // one operand, one stage: 32 KiB
constexpr int kSlot = 2 * kOp;                // A + W of one stage: 64 KiB
constexpr uint32_t kOOB = 0x80000000u;        // buffer offset past any range
constexpr int kLdsBytes = 2 * kSlot;

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

// A lane's 32-byte MFMA operand is kept as two 16-byte halves (the two LDS
// reads that fetch it may be issued at different points of the schedule).
struct Frags {
    uint4 a[4][2], b[4][2];
};

__device__ __forceinline__ v8i op(const uint4 (&h)[2])
{
    return v8i{(int)h[0].x, (int)h[0].y, (int)h[0].z, (int)h[0].w, (int)h[1].x, (int)h[1].y, (int)h[1].z, (int)h[1].w};
}

template <int EPI, int SMODE>
__global__ __launch_bounds__(kThreads, 1) void gemm_fp8_kernel(const GemmArgs g)
{
    __shared__ __attribute__((aligned(2048))) uint8_t lds[kLdsBytes];
    __shared__ __attribute__((aligned(16))) float lds_sa[kBM];
    __shared__ __attribute__((aligned(16))) float lds_sw[kBN];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const int wm = wave >> 1, wn = wave & 1;
    const Tile T = tile_of<EPI>(g);

    const uint8_t *A = g.A + (g.stride_a ? T.b * g.stride_a : 0);
    const uint8_t *W = g.W + (g.stride_w ? T.b * g.stride_w : 0);

    const int split = blockIdx.y;
    const int64_t k_begin = (int64_t)split * g.k_chunk;
    const int64_t k_end = min(g.K, k_begin + g.k_chunk);
    const int nk = (int)((k_end - k_begin + kBK - 1) / kBK);
    const int64_t Nh = g.N / 2;

    // scales into LDS (read by the epilogue after the main loop's barriers)
    stage_scales<EPI, SMODE>(g, T, lds_sa, lds_sw);

    // ---- copy setup -----------------------------------------------------------
    // Wave w fills tile rows [64 w, 64 w + 64) of A and of W: eight 8-row
    // blocks each, one 1 KiB copy instruction per block.  In a block lane L
    // owns LDS slot L: row L / 8, physical chunk L % 8, so it fetches logical
    // chunk (L % 8) ^ ((row >> 1) & 7); for 8-row blocks at row 64 w + 8 i
    // that XOR term is 4 (i & 1) + L / 16 (mod 8), so two offsets per operand
    // serve all eight blocks, the row step going into the scalar offset.
    const uint32_t rib = lane >> 3, pchunk = lane & 7;
    const uint32_t c_even = pchunk ^ ((lane >> 4) & 7u);
    const uint32_t c_odd = pchunk ^ ((4u + (lane >> 4)) & 7u);
    const int64_t a_rows = min((int64_t)kBM, g.M - T.m0);
    const v4i rs_a = make_rsrc(A + T.m0 * g.lda, (uint32_t)(a_rows * g.lda));
    // W: waves 0,1 the first 128 tile rows, waves 2,3 the second 128 (SWIGLU:
    // gate rows n0.., up rows N/2 + n0..)
    int64_t w_first, w_rows;
    if (EPI == SPG_EPI_SWIGLU) {
        w_rows = min((int64_t)128, Nh - T.n0);
        w_first = (wave < 2 ? T.n0 : Nh + T.n0);
    } else {
        const int64_t half0 = T.n0 + (wave < 2 ? 0 : 128);
        w_rows = min((int64_t)128, g.N - half0);
        w_first = half0;
    }
    w_rows = max(w_rows, (int64_t)0);
    const v4i rs_w = make_rsrc(W + w_first * g.ldw, (uint32_t)(w_rows * g.ldw));
    const uint32_t ra0 = (uint32_t)(wave * 64) + rib;            // A tile row of block 0
    const uint32_t rw0 = (uint32_t)((wave & 1) * 64) + rib;      // row within the W half
    const uint32_t va_e = ra0 * (uint32_t)g.lda + c_even * 16u, va_o = ra0 * (uint32_t)g.lda + c_odd * 16u;
    const uint32_t vw_e = rw0 * (uint32_t)g.ldw + c_even * 16u, vw_o = rw0 * (uint32_t)g.ldw + c_odd * 16u;
    const uint32_t lds_base =
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)&lds[0];

    // Copy instruction idx (0..15) of stage kt: 8-row block idx >> 1 of A
    // (idx even) or of W (idx odd).
    auto issue_one = [&](int kt, int idx) {
        const int i = idx >> 1;
        const int64_t k0 = k_begin + (int64_t)kt * kBK;
        const bool full = k0 + kBK <= k_end;
        const bool odd = i & 1;
        const bool in = full || (k0 + (int64_t)(odd ? c_odd : c_even) * 16 < k_end);
        const uint32_t la = (uint32_t)__builtin_amdgcn_readfirstlane(
            (int)(lds_base + (uint32_t)((kt & 1) * kSlot) + (uint32_t)(wave * 64 * kBK)));
        // The range check of a raw buffer access covers the VGPR offset only,
        // so the row step stays in the VGPR offset (rows past the valid range
        // then read as zero) and only k0, which never crosses a row, goes in
        // the scalar offset.
        const uint32_t soff = (uint32_t)__builtin_amdgcn_readfirstlane((int)k0);
        if ((idx & 1) == 0) {
            const uint32_t va = in ? (odd ? va_o : va_e) + (uint32_t)(8 * i) * (uint32_t)g.lda : kOOB;
            dma16(la + (uint32_t)(i * 8 * kBK), va, rs_a, soff);
        } else {
            const uint32_t vw = in ? (odd ? vw_o : vw_e) + (uint32_t)(8 * i) * (uint32_t)g.ldw : kOOB;
            dma16(la + (uint32_t)kOp + (uint32_t)(i * 8 * kBK), vw, rs_w, soff);
        }
    };
    auto issue_all = [&](int kt) {
        if (kt >= nk) return;
#pragma unroll
        for (int idx = 0; idx < 16; ++idx) issue_one(kt, idx);
    };

    // ---- fragment addressing ---------------------------------------------------
    // Fragment rows are 32-row aligned, so (row >> 1) & 7 depends on the lane
    // only: every fragment of a lane uses the same chunk offsets.
    const int l32 = lane & 31, khalf = lane >> 5;
    const uint32_t fx = ((uint32_t)l32 >> 1) & 7u;
    uint32_t foff[2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            foff[ks][h] = (uint32_t)l32 * kBK + ((((uint32_t)(ks * 4 + khalf * 2 + h)) ^ fx) << 4);
    auto brow0 = [&](int ni) -> uint32_t { return (uint32_t)wtile_row0<EPI>(wn, ni); };
    // Fragment half-reads r0 .. r1-1 of sub-step ks of stage kt: index 0..7
    // are the B fragments (ni = r / 2, half r % 2), 8..15 the A fragments.
    auto read_frags = [&](int kt, int ks, Frags &F, int r0, int r1) {
        const uint8_t *la = &lds[(kt & 1) * kSlot];
        const uint8_t *lb = la + kOp;
#pragma unroll
        for (int r = r0; r < r1; ++r) {
            const int h = r & 1;
            if (r < 8) {
                const int ni = r >> 1;
                F.b[ni][h] = *reinterpret_cast<const uint4 *>(lb + brow0(ni) * kBK + foff[ks][h]);
            } else {
                const int mi = (r - 8) >> 1;
                F.a[mi][h] = *reinterpret_cast<const uint4 *>(la + (uint32_t)(wm * 128 + mi * 32) * kBK + foff[ks][h]);
            }
        }
    };

    Acc acc;
    zero_acc(acc);

    // One stage = 32 MFMAs (sub-step 0 from F0, sub-step 1 from F1) in a
    // fixed order, with the other work of the stage slotted between them so
    // that the single wave per SIMD never stalls its MFMA issue for long:
    //   after MFMA 0..5   : the 16 fragment reads of F1 (sub-step 1, this stage)
    //   after MFMA 7      : F1 complete -> barrier: slot kt & 1 is free
    //   after MFMA 8..23  : one copy instruction each for stage kt + 2
    //   after MFMA 23     : own copy of stage kt + 1 landed -> barrier: published
    //   after MFMA 24..31 : the 16 fragment reads of F0 (sub-step 0, stage kt+1)
    Frags F0, F1;
    if (nk > 0) {
        issue_all(0);
        issue_all(1);
        if (nk > 1) wait_vmem<16>();
        else wait_vmem<0>();
        block_barrier();                       // stage 0 published
        read_frags(0, 0, F0, 0, 16);
        for (int kt = 0; kt < nk; ++kt) {
            const bool next = kt + 1 < nk, next2 = kt + 2 < nk;
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                const int mi = (j & 15) >> 2, ni = j & 3;
                const Frags &F = j < 16 ? F0 : F1;
                acc[ni][mi] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(op(F.b[ni]), op(F.a[mi]), acc[ni][mi],
                                                                              0, 0, 0, 0, 0, 0);
                if (j <= 5) read_frags(kt, 1, F1, j * 3, j == 5 ? 16 : j * 3 + 3);
                if (j == 7) {
                    wait_lds();
                    block_barrier();
                }
                if (j >= 8 && j <= 23 && next2) issue_one(kt + 2, j - 8);
                if (j == 23 && next) {
                    if (next2) wait_vmem<16>();
                    else wait_vmem<0>();
                    block_barrier();
                }
                if (j >= 24 && next) read_frags(kt + 1, 0, F0, (j - 24) * 2, (j - 24) * 2 + 2);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    __syncthreads();

    if (g.split_k > 1) {
        splitk_store(g, T, acc);      // the slices are summed by splitk_reduce_kernel
        return;
    }
    epilogue<EPI>(g, T, acc, lds_sa, lds_sw, &lds[(threadIdx.x >> 6) * 32768]);   // after the barrier above
}

template <int EPI>
hipError_t launch_epi(const GemmArgs &g, const spg_plan &p, hipStream_t s)
{
    dim3 grid((unsigned)p.tiles, (unsigned)g.split_k, 1);
    if (g.format == SPG_FMT_E4M3_ROW)
        gemm_fp8_kernel<EPI, SPG_FMT_E4M3_ROW><<<grid, kThreads, 0, s>>>(g);
    else
        gemm_fp8_kernel<EPI, SPG_FMT_E4M3_TENSOR><<<grid, kThreads, 0, s>>>(g);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && g.split_k > 1) e = launch_splitk_reduce(g, p.tiles, s);
    return e;
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
