// FP8 E4M3 scaled GEMM for gfx950 with fused bf16 epilogues.
//
// out = epilogue(s_a * s_w * sum_k a_k w_k), A [M,K] and W [N,K] K-contiguous
// (the NT layout of AstrAI's per-tensor E4M3 benchmark), fp32
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
//    registers ("slot free": the copy of stage kt+2 starts), and after MFMA
//    19 ("stage kt+1 published": its first fragments are read while the last
//    12 MFMAs run).  A copy has between 21 and 43 MFMAs to land.
//  * SWIGLU pairs weight rows inside one 256-row W tile (128 gate + 128 up).
//  * XCD-aware tile order; a persistent grid (one workgroup per compute
//    unit) whose copy pipeline runs on into the next tile; optional split-K
//    through the workspace; a half-height kernel (128-row tiles) for a short
//    last round and for whole products where the route model prices 128-row
//    tiles below 256-row ones.
//  * Epilogue from the accumulators, transposed through a per-wave LDS region
//    so the output leaves in whole 128-byte row segments (W fragments are the
//    first MFMA operand, so a lane holds four adjacent output columns).
//  * Few-token products split along K (at most 64 tokens) use instantiations
//    that leave out the MFMAs of the empty A blocks.
#include "spg_gemm_common.h"

#include <type_traits>

namespace spg {

namespace {

using namespace gemm;
constexpr int kBK = 128;                      // K bytes (E4M3 elements) per stage
constexpr int kOp = kBM * kBK;                // one operand, one stage: 32 KiB
constexpr int kSlot = 2 * kOp;                // A + W of one stage: 64 KiB

// A lane's 32-byte MFMA operand is kept as two 16-byte halves (the two LDS
// reads that fetch it may be issued at different points of the schedule).
struct Frags {
    uint4 a[4][2], b[4][2];
};

__device__ __forceinline__ v8i op(const uint4 (&h)[2])
{
    return v8i{(int)h[0].x, (int)h[0].y, (int)h[0].z, (int)h[0].w, (int)h[1].x, (int)h[1].y, (int)h[1].z, (int)h[1].w};
}

// Copy sources of one tile: buffer resources over its A rows and its two
// 128-row W halves (each wave copies 64 rows of A and 64 rows of one W half).
struct CopySrc {
    v4i a, w;
};

// AM: A blocks per wave that take part in the MFMAs.  4 in general; 1 (2)
// for products of at most 32 (64) tokens, where only the first 32 (64) rows
// of a tile exist: the MFMAs (and fragment reads) of the empty blocks are
// left out, so the stage is paced by the weight copies instead of 32 MFMAs on
// zeros (the waves of the lower half compute the zero blocks of their rows,
// which keeps all four waves equally busy).
// SO: the output is column segments (a separate instantiation, see epilogue).
template <int EPI, int SMODE, bool SPLIT, int AM = 4, bool SO = false>
__global__ __launch_bounds__(kThreads, 1) void gemm_fp8_kernel(const GemmArgs g)
{
    __shared__ __attribute__((aligned(2048))) uint8_t lds[2 * kSlot + kEpiRegionBytes];
    // Row-wise SWIGLU copies the scale factors straight into LDS, into a ring
    // of three buffers (see below); the other forms load them into registers
    // a tile ahead and store them into two alternating buffers.
    constexpr bool kScaleDma = !SPLIT && EPI == SPG_EPI_SWIGLU && SMODE == SPG_FMT_E4M3_ROW;
    constexpr int kScaleBufs = kScaleDma ? 3 : 2;
    __shared__ __attribute__((aligned(16))) float lds_scale[kScaleBufs][2][kBM];   // [buffer][a / w][row]
    __shared__ __attribute__((aligned(16))) float lds_bias[bias_words<EPI>()];
    clock_mark(g.clocks, 0);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const int wm = wave >> 1, wn = wave & 1;

    // Tiles of this workgroup: virtual workgroup ids blockIdx.x + i * gridDim.x
    // (a persistent grid of one workgroup per compute unit walks the same
    // XCD-aware order a one-tile-per-workgroup launch would).
    // A split launch has one workgroup per (tile, K slice) work item.
    const int64_t total = g.tile_count;
    const WorkItem wi = SPLIT ? work_item(g) : WorkItem{0, 0};
    const int ntile = SPLIT ? 1 : (int)((total - (int64_t)blockIdx.x + gridDim.x - 1) / gridDim.x);
    auto tile_i = [&](int i) -> Tile {
        if (SPLIT) return tile_from_id<EPI>(g, g.tile_begin + wi.tile);
        return tile_from_id<EPI>(g, g.tile_begin + xcd_remap((int64_t)blockIdx.x + (int64_t)i * gridDim.x, total));
    };

    // (unsplit: blockIdx.y is 0; kept as a run-time value because folding
    // the constant changes the register allocation of the whole kernel and
    // measured 13% slower on 4096 x 34816 x 5120)
    const int split = SPLIT ? wi.split : (int)blockIdx.y;
    const int64_t k_begin = (int64_t)split * g.k_chunk;
    const int64_t k_end = min(g.K, k_begin + g.k_chunk);
    const int nk = (int)((k_end - k_begin + kBK - 1) / kBK);
    const int64_t Nh = g.N / 2;

    // ---- copy setup -----------------------------------------------------------
    // Wave w fills tile rows [64 w, 64 w + 64) of A and of W: eight 8-row
    // blocks each, one 1 KiB copy instruction per block.  In a block lane L
    // owns LDS slot L: row L / 8, physical chunk L % 8, so it fetches logical
    // chunk (L % 8) ^ ((row >> 1) & 7); for 8-row blocks at row 64 w + 8 i
    // that XOR term is 4 (i & 1) + L / 16 (mod 8), so two offsets per operand
    // serve all eight blocks.
    auto make_src = [&](const Tile &T) -> CopySrc {
        const uint8_t *A = g.A + (g.stride_a ? T.b * g.stride_a : 0);
        const uint8_t *W = g.W + (g.stride_w ? T.b * g.stride_w : 0);
        const int64_t a_rows = min((int64_t)kBM, g.M - T.m0);
        // W: waves 0,1 the first 128 tile rows, waves 2,3 the second 128
        // (SWIGLU: gate rows n0.., up rows N/2 + n0..)
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
        return CopySrc{make_rsrc(A + T.m0 * g.lda, (uint32_t)(a_rows * g.lda)),
                       make_rsrc(W + w_first * g.ldw, (uint32_t)(w_rows * g.ldw))};
    };
    // Lane-dependent copy and fragment offsets.  They are recomputed for every
    // tile from an opaque copy of the lane id, so that they are dead (not
    // kept in registers, nor spilled) while a tile's epilogue runs.
    struct LaneCtx {
        uint32_t c_even, c_odd, va_e, va_o, vw_e, vw_o;
        uint32_t foff[2][2];
    };
    auto lane_ctx = [&]() -> LaneCtx {
        const int ln = lane_id();
        LaneCtx c;
        const uint32_t rib = (uint32_t)ln >> 3, pchunk = (uint32_t)ln & 7;
        c.c_even = pchunk ^ (((uint32_t)ln >> 4) & 7u);
        c.c_odd = pchunk ^ ((4u + ((uint32_t)ln >> 4)) & 7u);
        const uint32_t ra0 = (uint32_t)(wave * 64) + rib;        // A tile row of block 0
        const uint32_t rw0 = (uint32_t)((wave & 1) * 64) + rib;  // row within the W half
        c.va_e = ra0 * (uint32_t)g.lda + c.c_even * 16u;
        c.va_o = ra0 * (uint32_t)g.lda + c.c_odd * 16u;
        c.vw_e = rw0 * (uint32_t)g.ldw + c.c_even * 16u;
        c.vw_o = rw0 * (uint32_t)g.ldw + c.c_odd * 16u;
        // Fragment rows are 32-row aligned, so (row >> 1) & 7 depends on the
        // lane only: every fragment of a lane uses the same chunk offsets.
        const uint32_t l32 = (uint32_t)ln & 31, khalf = (uint32_t)ln >> 5;
        const uint32_t fx = (l32 >> 1) & 7u;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                c.foff[ks][h] = l32 * kBK + ((((uint32_t)ks * 4 + khalf * 2 + (uint32_t)h) ^ fx) << 4);
        return c;
    };
    LaneCtx L = lane_ctx();
    const uint32_t lds_base =
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)&lds[0];

    // Per-stage copy plan: source tile, scalar K offset and the per-lane base
    // offsets of the even / odd 8-row blocks (kOOB where a lane's 16 bytes lie
    // past K, or for a stage that does not exist: such copies read zeros into
    // a slot nobody reads again, which keeps every wait count uniform).
    struct StageCopy {
        v4i ra, rw;
        uint32_t soff, a_e, a_o, w_e, w_o;
    };
    auto plan_stage = [&](const CopySrc &src, int kt, bool exists) -> StageCopy {
        const int64_t k0 = k_begin + (int64_t)kt * kBK;
        const bool full = k0 + kBK <= k_end;
        const bool in_e = exists && (full || k0 + (int64_t)L.c_even * 16 < k_end);
        const bool in_o = exists && (full || k0 + (int64_t)L.c_odd * 16 < k_end);
        // The range check of a raw buffer access covers the VGPR offset only,
        // so the row step stays in the VGPR offset (rows past the valid range
        // then read as zero) and only k0, which never crosses a row, goes in
        // the scalar offset.
        StageCopy c;
        c.ra = src.a;
        c.rw = src.w;
        c.soff = (uint32_t)__builtin_amdgcn_readfirstlane((int)(exists ? k0 : 0));
        c.a_e = in_e ? L.va_e : kOOB;
        c.a_o = in_o ? L.va_o : kOOB;
        c.w_e = in_e ? L.vw_e : kOOB;
        c.w_o = in_o ? L.vw_o : kOOB;
        return c;
    };
    // Copy instruction idx (0..15) of a stage into LDS slot `slot`: 8-row
    // block idx >> 1 of A (idx even) or of W (idx odd).  kOOB plus the row
    // step stays past any buffer range (ranges are at most 2^31 bytes).
    auto issue_one = [&](const StageCopy &c, int slot, int idx) {
        const int i = idx >> 1;
        const bool odd = i & 1;
        const uint32_t la = (uint32_t)__builtin_amdgcn_readfirstlane(
            (int)(lds_base + (uint32_t)(slot * kSlot) + (uint32_t)(wave * 64 * kBK)));
        if ((idx & 1) == 0)
            dma16(la + (uint32_t)(i * 8 * kBK), (odd ? c.a_o : c.a_e) + (uint32_t)(8 * i) * (uint32_t)g.lda, c.ra, c.soff);
        else
            dma16(la + (uint32_t)kOp + (uint32_t)(i * 8 * kBK), (odd ? c.w_o : c.w_e) + (uint32_t)(8 * i) * (uint32_t)g.ldw,
                  c.rw, c.soff);
    };

    // ---- fragment addressing ---------------------------------------------------
    auto brow0 = [&](int ni) -> uint32_t { return (uint32_t)wtile_row0<EPI>(wn, ni); };
    // Fragment half-reads r0 .. r1-1 of sub-step ks from LDS slot `slot`:
    // index 0..7 are the W fragments (ni = r / 2, half r % 2), 8..15 the A
    // fragments.
    auto read_frags = [&](int slot, int ks, Frags &F, int r0, int r1) {
        const uint8_t *la = &lds[slot * kSlot];
        const uint8_t *lb = la + kOp;
        // A fixed 16-trip loop with the range as a condition: it unrolls before
        // the schedule's loop does, so every fragment index is a constant (a
        // loop over r0 .. r1 can stay rolled, and then the fragment registers
        // are indexed at run time, i.e. kept in scratch memory).
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            if (r < r0 || r >= r1) continue;
            const int h = r & 1;
            if (r < 8) {
                const int ni = r >> 1;
                F.b[ni][h] = *reinterpret_cast<const uint4 *>(lb + brow0(ni) * kBK + L.foff[ks][h]);
            } else {
                const int mi = (r - 8) >> 1;
                F.a[mi][h] = *reinterpret_cast<const uint4 *>(la + (uint32_t)(wm * 128 + mi * 32) * kBK + L.foff[ks][h]);
            }
        }
    };

    // Scale factors of tile T into lds_scale[buf] by direct copies (row-wise
    // SWIGLU): tile row r = 64 wave + lane.  A: token row m0 + r (zero past
    // M).  W: gate row n0 + r for r < 128, up row N/2 + n0 + r - 128 above
    // (zero where n0 + (r mod 128) >= N/2); the same rows make_src copies.
    // The lane offsets come from an opaque lane id, so nothing derived from
    // threadIdx.x stays live (or spilled) across the tile loop.
    auto issue_scales = [&](const Tile &T, int buf) {
        const uint32_t ln = (uint32_t)lane_id();
        const float *sa = (const float *)g.sa + (g.stride_a ? T.b * g.sa_bstride : 0) + T.m0;
        const float *sw = (const float *)g.sw + (g.stride_w ? T.b * g.sw_bstride : 0);
        const int64_t a_rows = max((int64_t)0, min((int64_t)kBM, g.M - T.m0));
        const int64_t w_rows = max((int64_t)0, min((int64_t)128, Nh - T.n0));
        const int64_t w_first = wave < 2 ? T.n0 : Nh + T.n0;
        const uint32_t la = (uint32_t)__builtin_amdgcn_readfirstlane(
            (int)(uint32_t)(uintptr_t)(const __attribute__((address_space(3))) float *)&lds_scale[buf][0][wave * 64]);
        const uint32_t lw = (uint32_t)__builtin_amdgcn_readfirstlane(
            (int)(uint32_t)(uintptr_t)(const __attribute__((address_space(3))) float *)&lds_scale[buf][1][wave * 64]);
        dma4(la, ((uint32_t)(wave * 64) + ln) * 4u, make_rsrc(sa, (uint32_t)(a_rows * 4)), 0);
        dma4(lw, ((uint32_t)((wave & 1) * 64) + ln) * 4u, make_rsrc(sw + w_first, (uint32_t)(w_rows * 4)), 0);
    };

    Tile Tc = tile_i(0), Tn = Tc;
    CopySrc sc = make_src(Tc), sn = sc;
    bool has_next = ntile > 1;
    if (has_next) {
        Tn = tile_i(1);
        sn = make_src(Tn);
    }
    if constexpr (kScaleDma) {
        // tiles 0 and 1; both land before the first stage is published
        issue_scales(Tc, 0);
        if (has_next) issue_scales(Tn, 1);
    } else {
        stage_scales<EPI, SMODE>(g, Tc, lds_scale[0][0], lds_scale[0][1]);
    }

    // One stage = 32 MFMAs (sub-step 0 from F0, sub-step 1 from F1) in a
    // fixed order, with the other work of the stage slotted between them so
    // that the single wave per SIMD never stalls its MFMA issue for long:
    //   after MFMA 0..5   : the 16 fragment reads of F1 (sub-step 1, this stage)
    //   after MFMA 7      : F1 complete -> barrier: the stage's slot is free
    //   after MFMA 8..30  : the 16 copy instructions for the stage after next,
    //                       two in every three MFMAs (at 8 + floor(3 i / 2))
    //   after MFMA 19     : own copy of the next stage landed -> barrier: published
    //   after MFMA 20..31 : the 16 fragment reads of F0 (sub-step 0, next stage)
    // Spreading the copies over 24 MFMAs instead of 16 keeps the memory path's
    // issue queue from filling (measured: steady stage 2565 -> 2470 cycles
    // against the 2048 of the MFMAs alone).
    // "Next" runs on into the following tile of the workgroup, whose first two
    // stages are thus copied during the last two stages of the current tile
    // and land while its epilogue runs.  Stages alternate between the two
    // slots over the whole sequence (parity G).
    Frags F0, F1;
    {
        // stages 0 and 1 of the sequence (stage 1 is the next tile's first
        // when this tile has a single stage)
        const StageCopy c0 = plan_stage(sc, 0, nk > 0);
        const StageCopy c1 = nk > 1 ? plan_stage(sc, 1, true) : plan_stage(sn, 0, has_next);
#pragma unroll
        for (int idx = 0; idx < 16; ++idx) issue_one(c0, 0, idx);
#pragma unroll
        for (int idx = 0; idx < 16; ++idx) issue_one(c1, 1, idx);
        wait_vmem<16>();
        block_barrier();                       // stage 0 published
        read_frags(0, 0, F0, 0, 16);
    }
    int G = 0;                                 // stage counter over all tiles (slot = G & 1)
    // One stage; the last stage of a tile does not prefetch the next stage's
    // F0 (it is read after the epilogue, so no fragment registers are live
    // across it).
    auto stage = [&](Acc &acc, int kt, auto last_c) {
        constexpr bool LAST = decltype(last_c)::value;
        const int slot = G & 1;
        // stage G + 2: this tile's kt + 2, else the next tile's kt + 2 - nk
        const bool here = kt + 2 < nk;
        const StageCopy c2 = plan_stage(here ? sc : sn, here ? kt + 2 : kt + 2 - nk,
                                        here || (has_next && kt + 2 - nk < nk));
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            const int mi = (j & 15) >> 2, ni = j & 3;
            const Frags &F = j < 16 ? F0 : F1;
            if (mi < AM)
                acc[ni][mi] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(op(F.b[ni]), op(F.a[mi]), acc[ni][mi],
                                                                              0, 0, 0, 0, 0, 0);
            if (j <= 5) read_frags(slot, 1, F1, j * 3, j == 5 ? 16 : j * 3 + 3);
            if (j == 7) {
                wait_lds();
                block_barrier();
            }
            // The wave's eight A blocks first, then its eight W blocks.  An A
            // line is shared by the four tiles of a tile row in flight on an
            // XCD and a W line by eight, so A copies miss the L2 more often;
            // returns are in order, so a miss delays every later copy of the
            // wave, and issuing the A copies first gives their misses the
            // longest time to land (measured on 4096 x 34816 x 5120: 3% fewer
            // cycles than alternating A and W).
#pragma unroll
            for (int ci = 0; ci < 16; ++ci)
                if (j == 8 + (3 * ci) / 2) issue_one(c2, slot, ci < 8 ? 2 * ci : 2 * (ci - 8) + 1);
            if (j == 19) {
                // copies 0..7 of stage G + 2 are issued by now (j <= 19)
                wait_vmem<8>();                // stage G + 1 landed (stage G + 2 in flight)
                block_barrier();
            }
            if (!LAST && j >= 20) read_frags(slot ^ 1, 0, F0, (j - 20) * 4 / 3, (j - 19) * 4 / 3);
            __builtin_amdgcn_sched_barrier(0);
        }
        ++G;
    };
    for (int i = 0; i < ntile; ++i) {
        // The next tile's scale factors are loaded now, a whole tile before
        // they are written to LDS: loads and stores share the vector-memory
        // counter, so loading them next to this tile's output stores would
        // make every wave's wait for them wait for its stores too (and for
        // the loads' own latency).
        float nsa = 0.0f, nsw = 0.0f;
        if (!kScaleDma && i + 1 < ntile) scale_values<EPI, SMODE>(g, Tn, nsa, nsw);
        Acc acc;
        zero_acc(acc);
        for (int kt = 0; kt + 1 < nk; ++kt) stage(acc, kt, std::false_type{});
        if (nk > 0) stage(acc, nk - 1, std::true_type{});

        if constexpr (kScaleDma) {
            // The scales of tile i + 2 go into buffer (i + 2) mod 3 now, so
            // their copies land while this epilogue runs.  That buffer last
            // held tile i - 1's scales: every wave has passed a barrier of
            // tile i (the one below when K is empty) since its epilogue of
            // tile i - 1.  The copies are complete (by the stage waits, or the
            // wait below) and published by a barrier before tile i + 2's
            // epilogue reads them.
            if (nk == 0) {
                wait_vmem<0>();
                block_barrier();
            }
            if (i + 2 < ntile) issue_scales(tile_i(i + 2), (i + 2) % 3);
        }
        if (SPLIT) {
            splitk_store(g, Tc, split, acc);   // the slices are summed by splitk_reduce_kernel
        } else {
            // SWIGLU is given the wave index computed above: re-deriving it
            // from threadIdx.x lets the compiler keep a per-lane copy live
            // across the tile loop and spill it, and the reload's wait on the
            // vector memory counter also waits for the next tile's copies in
            // flight (measured: 1-2% of the 4096 x 34816 x 5120 product).  The
            // other epilogues measured slightly faster re-deriving it.
            const int sb = kScaleDma ? i % 3 : i & 1;
            epilogue<EPI, 4, EPI == SPG_EPI_SWIGLU, false, SO>(g, Tc, acc, lds_scale[sb][0], lds_scale[sb][1], lds_bias,
                                                   &lds[2 * kSlot + wave * (kEpiRegionBytes / 4)], wave);
        }
        if (i + 1 < ntile) {
            L = lane_ctx();
            read_frags(G & 1, 0, F0, 0, 16);   // the next tile's stage 0, published at the last barrier
            Tc = Tn;
            sc = sn;
            has_next = i + 2 < ntile;
            if (has_next) {
                Tn = tile_i(i + 2);
                sn = make_src(Tn);
            }
            // Every wave has passed this tile's barriers, so none still reads
            // the scales of tile i - 1 that share this buffer.
            if (!kScaleDma) {
                const int t = wave * 64 + lane_id();
                lds_scale[(i + 1) & 1][0][t] = nsa;
                lds_scale[(i + 1) & 1][1][t] = nsw;
            }
        }
    }
    wait_vmem<0>();   // no copy into LDS may still be in flight when the workgroup ends
    clock_mark(g.clocks, 1);
}

// ---------------------------------------------------------------------------
// Half-height tiles (128 x 256), one per workgroup.  Two uses: a short last
// round (when the tiles leave a last round that fills at most half of the
// compute units - 4096 x 34816 x 5120 SwiGLU: 2176 tiles = 8.5 rounds of 256
// - those tiles run in a second launch as 128 x 256 halves, so the round is
// spread over every compute unit and takes about half as long; unlike a K
// split this needs no partial tiles and no reduction), and whole products
// over a grid of 128-row tiles: 65 - 128 tokens, where a full tile's lower
// half would hold no rows, and where the planner's route model prefers
// 128-row tiles.  A tail half whose rows all lie past M returns at once.
//
// Same data path as the full kernel (direct-to-LDS copies of 128-byte row
// segments, the same swizzle, W fragments first), with the A side halved:
// waves (wm, wn) hold 64 token rows x 128 weight rows (2 x 4 blocks of
// 32x32), and a stage is 16 MFMAs.  A stage of the slot holds 128 A rows
// (16 KiB) and 256 W rows (32 KiB); three slots, so a copy is issued two
// stages ahead of its use and still has ~25 MFMAs to land, and one barrier
// per stage both frees the current slot and publishes the next.  Per stage:
//   after MFMA 0..3   : the 12 fragment reads of F1 (sub-step 1)
//   after MFMA 5      : F1 complete and the next stage landed -> barrier
//   after MFMA 6..13  : the 12 copies of the stage three ahead into this slot
//   after MFMA 8..11  : the 12 fragment reads of F0 of the next stage (F0's
//                       last MFMA is 7)
// ---------------------------------------------------------------------------
constexpr int kHalfRows = 128;                     // A rows of a half tile
constexpr int kOpAh = kHalfRows * kBK;             // A bytes of one stage: 16 KiB
constexpr int kSlotH = kOpAh + kOp;                // A + W of one stage: 48 KiB
constexpr int kSlotsH = 3;
static_assert(4 * 16384 <= kSlotsH * kSlotH, "the epilogue's staged regions fit in the freed slots");

struct FragsH {
    uint4 a[2][2], b[4][2];
};

template <int EPI, int SMODE, bool SO = false>
__global__ __launch_bounds__(kThreads, 1) void gemm_fp8_half_kernel(const GemmArgs g)
{
    __shared__ __attribute__((aligned(2048))) uint8_t lds[kSlotsH * kSlotH];
    __shared__ __attribute__((aligned(16))) float lds_sa[kBM];
    __shared__ __attribute__((aligned(16))) float lds_sw[kBN];
    __shared__ __attribute__((aligned(16))) float lds_bias[bias_words<EPI>()];
    clock_mark(g.clocks, 0);

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;

    // work item v: over a grid of 128-row tiles, tile v; else half v & 1 of
    // 256-row tile tile_begin + v / 2 (the two halves of a tile are
    // neighbours in the XCD-aware order and share its W panel)
    const bool grid128 = g.rows128 != 0;
    const uint32_t v = (uint32_t)xcd_remap(blockIdx.x, (grid128 ? 1 : 2) * g.tile_count);
    Tile T;
    if (grid128) {
        T = tile_from_id<EPI, kHalfRows>(g, g.tile_begin + v);
    } else {
        T = tile_from_id<EPI>(g, g.tile_begin + (v >> 1));
        T.m0 += (int64_t)(v & 1u) * kHalfRows;
    }
    if (T.m0 >= g.M) return;                       // lower half of a ragged last tile row

    // The scale factors are written to LDS after the main loop: a wait the
    // compiler inserts for these loads would also wait for every copy.
    float va, vw;
    scale_values<EPI, SMODE>(g, T, va, vw);

    const int nk = (int)((g.K + kBK - 1) / kBK);
    const int64_t Nh = g.N / 2;

    // ---- copy setup (as the full kernel; wave w copies A rows 32 w .. 32 w + 31
    // in four 8-row blocks and W rows 64 w .. 64 w + 63 in eight) -------------
    const uint8_t *A = g.A + (g.stride_a ? T.b * g.stride_a : 0);
    const uint8_t *W = g.W + (g.stride_w ? T.b * g.stride_w : 0);
    const int64_t a_rows = min((int64_t)kHalfRows, g.M - T.m0);
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
    const v4i rs_a = make_rsrc(A + T.m0 * g.lda, (uint32_t)(a_rows * g.lda));
    const v4i rs_w = make_rsrc(W + w_first * g.ldw, (uint32_t)(w_rows * g.ldw));
    const int ln = lane_id();
    const uint32_t rib = (uint32_t)ln >> 3, pchunk = (uint32_t)ln & 7;
    // 8-row blocks start at multiples of 8 rows, so the swizzle term of a
    // lane is 4 (block & 1) + lane / 16 (mod 8), for A (rows 32 w + 8 i) as
    // for W (rows 64 w + 8 i)
    const uint32_t c_even = pchunk ^ (((uint32_t)ln >> 4) & 7u);
    const uint32_t c_odd = pchunk ^ ((4u + ((uint32_t)ln >> 4)) & 7u);
    const uint32_t ra0 = (uint32_t)(wave * 32) + rib;
    const uint32_t rw0 = (uint32_t)((wave & 1) * 64) + rib;
    const uint32_t va_e = ra0 * (uint32_t)g.lda + c_even * 16u, va_o = ra0 * (uint32_t)g.lda + c_odd * 16u;
    const uint32_t vw_e = rw0 * (uint32_t)g.ldw + c_even * 16u, vw_o = rw0 * (uint32_t)g.ldw + c_odd * 16u;
    const uint32_t lds_base =
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)&lds[0];

    struct StageCopy {
        uint32_t soff, a_e, a_o, w_e, w_o;
    };
    // offsets of stage kt; kOOB for bytes past K and for stages past the end
    // (zeros into a slot nobody reads again: every wait count stays uniform)
    auto plan_stage = [&](int kt) -> StageCopy {
        const bool exists = kt < nk;
        const int64_t k0 = (int64_t)kt * kBK;
        const bool full = k0 + kBK <= g.K;
        const bool in_e = exists && (full || k0 + (int64_t)c_even * 16 < g.K);
        const bool in_o = exists && (full || k0 + (int64_t)c_odd * 16 < g.K);
        StageCopy c;
        c.soff = (uint32_t)__builtin_amdgcn_readfirstlane((int)(exists ? k0 : 0));
        c.a_e = in_e ? va_e : kOOB;
        c.a_o = in_o ? va_o : kOOB;
        c.w_e = in_e ? vw_e : kOOB;
        c.w_o = in_o ? vw_o : kOOB;
        return c;
    };
    // copy instruction idx (0..11) of a stage: W, W, A, W, W, A, ... (W blocks
    // 0..7, A blocks 0..3)
    auto issue_one = [&](const StageCopy &c, int slot, int idx) {
        const uint32_t sb = lds_base + (uint32_t)(slot * kSlotH);
        if (idx % 3 == 2) {
            const int i = idx / 3;
            const uint32_t la = (uint32_t)__builtin_amdgcn_readfirstlane(
                (int)(sb + (uint32_t)(wave * 32 * kBK) + (uint32_t)(i * 8 * kBK)));
            dma16(la, ((i & 1) ? c.a_o : c.a_e) + (uint32_t)(8 * i) * (uint32_t)g.lda, rs_a, c.soff);
        } else {
            const int i = (idx / 3) * 2 + (idx % 3);
            const uint32_t la = (uint32_t)__builtin_amdgcn_readfirstlane(
                (int)(sb + (uint32_t)kOpAh + (uint32_t)(wave * 64 * kBK) + (uint32_t)(i * 8 * kBK)));
            dma16(la, ((i & 1) ? c.w_o : c.w_e) + (uint32_t)(8 * i) * (uint32_t)g.ldw, rs_w, c.soff);
        }
    };

    // ---- fragments: reads 0..7 are the W halves, 8..11 the A halves -----------
    const uint32_t l32 = (uint32_t)ln & 31, khalf = (uint32_t)ln >> 5, fx = (l32 >> 1) & 7u;
    uint32_t foff[2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            foff[ks][h] = l32 * kBK + ((((uint32_t)ks * 4 + khalf * 2 + (uint32_t)h) ^ fx) << 4);
    auto read_frags = [&](int slot, int ks, FragsH &F, int r0, int r1) {
        const uint8_t *la = &lds[slot * kSlotH];
        const uint8_t *lb = la + kOpAh;
#pragma unroll
        for (int r = 0; r < 12; ++r) {
            if (r < r0 || r >= r1) continue;
            const int h = r & 1;
            if (r < 8) {
                const int ni = r >> 1;
                F.b[ni][h] = *reinterpret_cast<const uint4 *>(lb + (uint32_t)wtile_row0<EPI>(wn, ni) * kBK + foff[ks][h]);
            } else {
                const int mi = (r - 8) >> 1;
                F.a[mi][h] = *reinterpret_cast<const uint4 *>(la + (uint32_t)(wm * 64 + mi * 32) * kBK + foff[ks][h]);
            }
        }
    };

    FragsH F0, F1;
    {
        const StageCopy c0 = plan_stage(0), c1 = plan_stage(1), c2 = plan_stage(2);
#pragma unroll
        for (int idx = 0; idx < 12; ++idx) issue_one(c0, 0, idx);
#pragma unroll
        for (int idx = 0; idx < 12; ++idx) issue_one(c1, 1, idx);
#pragma unroll
        for (int idx = 0; idx < 12; ++idx) issue_one(c2, 2, idx);
        wait_vmem<24>();                           // stage 0 landed (and the scale loads)
        block_barrier();
        read_frags(0, 0, F0, 0, 12);
    }

    Acc acc;                                       // blocks acc[x][0..1] are used
    zero_acc(acc);
    int slot = 0;                                  // slot of stage kt = kt % 3
    auto stage = [&](int kt, auto last_c) {
        constexpr bool LAST = decltype(last_c)::value;
        const int next = slot == 2 ? 0 : slot + 1;
        const StageCopy c3 = plan_stage(kt + 3);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int mi = (j & 7) >> 2, ni = j & 3;
            const FragsH &F = j < 8 ? F0 : F1;
            acc[ni][mi] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(op(F.b[ni]), op(F.a[mi]), acc[ni][mi],
                                                                          0, 0, 0, 0, 0, 0);
            if (j <= 3) read_frags(slot, 1, F1, j * 3, j * 3 + 3);
            if (j == 5) {
                // in flight: stages kt + 1 and kt + 2 (12 copies each, oldest
                // first); stage kt + 3 is not issued yet
                wait_lds();
                wait_vmem<12>();
                block_barrier();                   // this slot is free, stage kt + 1 published
            }
#pragma unroll
            for (int ci = 0; ci < 12; ++ci)
                if (j == 6 + (2 * ci) / 3) issue_one(c3, slot, ci);
            if (!LAST && j >= 8 && j <= 11) read_frags(next, 0, F0, (j - 8) * 3, (j - 8) * 3 + 3);
            __builtin_amdgcn_sched_barrier(0);
        }
        slot = next;
    };
    for (int kt = 0; kt + 1 < nk; ++kt) stage(kt, std::false_type{});
    if (nk > 0) stage(nk - 1, std::true_type{});

    // no copy may still be landing in LDS: the epilogue's staging region
    // overlaps the slots
    wait_vmem<0>();
    lds_sa[tid] = va;
    lds_sw[tid] = vw;
    block_barrier();
    // 16 KiB per wave of the freed slots: one region per pass
    epilogue<EPI, 2, false, true, SO>(g, T, acc, lds_sa, lds_sw, lds_bias, &lds[wave * 16384]);
    clock_mark(g.clocks, 1);
}

template <int EPI>
hipError_t launch_half(const GemmArgs &g, hipStream_t s)
{
    const dim3 grid((unsigned)((g.rows128 ? 1 : 2) * g.tile_count));
    const bool so = g.nseg != 0;
    if (g.format == SPG_FMT_E4M3_ROW) {
        if (so) gemm_fp8_half_kernel<EPI, SPG_FMT_E4M3_ROW, true><<<grid, kThreads, 0, s>>>(g);
        else gemm_fp8_half_kernel<EPI, SPG_FMT_E4M3_ROW><<<grid, kThreads, 0, s>>>(g);
    } else {
        if (so) gemm_fp8_half_kernel<EPI, SPG_FMT_E4M3_TENSOR, true><<<grid, kThreads, 0, s>>>(g);
        else gemm_fp8_half_kernel<EPI, SPG_FMT_E4M3_TENSOR><<<grid, kThreads, 0, s>>>(g);
    }
    return hipGetLastError();
}

template <int EPI>
hipError_t launch_epi(const GemmArgs &g, const spg_plan &p, hipStream_t s)
{
    // p.workgroups: one per (tile, slice) work item, or a persistent grid of
    // at most one per compute unit for unsplit products with two or more K
    // stages.
    const dim3 grid((unsigned)p.workgroups);
    const bool split = g.split_k > 1, so = g.nseg != 0;
    if (g.M <= 32) {
        // at most 32 tokens: one active A block per wave
        if (g.format == SPG_FMT_E4M3_ROW) {
            if (split) gemm_fp8_kernel<EPI, SPG_FMT_E4M3_ROW, true, 1><<<grid, kThreads, 0, s>>>(g);
            else if (so) gemm_fp8_kernel<EPI, SPG_FMT_E4M3_ROW, false, 1, true><<<grid, kThreads, 0, s>>>(g);
            else gemm_fp8_kernel<EPI, SPG_FMT_E4M3_ROW, false, 1><<<grid, kThreads, 0, s>>>(g);
        } else {
            if (split) gemm_fp8_kernel<EPI, SPG_FMT_E4M3_TENSOR, true, 1><<<grid, kThreads, 0, s>>>(g);
            else if (so) gemm_fp8_kernel<EPI, SPG_FMT_E4M3_TENSOR, false, 1, true><<<grid, kThreads, 0, s>>>(g);
            else gemm_fp8_kernel<EPI, SPG_FMT_E4M3_TENSOR, false, 1><<<grid, kThreads, 0, s>>>(g);
        }
    } else if (g.M <= 64) {
        // at most 64 tokens: two active A blocks per wave
        if (g.format == SPG_FMT_E4M3_ROW) {
            if (split) gemm_fp8_kernel<EPI, SPG_FMT_E4M3_ROW, true, 2><<<grid, kThreads, 0, s>>>(g);
            else if (so) gemm_fp8_kernel<EPI, SPG_FMT_E4M3_ROW, false, 2, true><<<grid, kThreads, 0, s>>>(g);
            else gemm_fp8_kernel<EPI, SPG_FMT_E4M3_ROW, false, 2><<<grid, kThreads, 0, s>>>(g);
        } else {
            if (split) gemm_fp8_kernel<EPI, SPG_FMT_E4M3_TENSOR, true, 2><<<grid, kThreads, 0, s>>>(g);
            else if (so) gemm_fp8_kernel<EPI, SPG_FMT_E4M3_TENSOR, false, 2, true><<<grid, kThreads, 0, s>>>(g);
            else gemm_fp8_kernel<EPI, SPG_FMT_E4M3_TENSOR, false, 2><<<grid, kThreads, 0, s>>>(g);
        }
    } else if (g.format == SPG_FMT_E4M3_ROW) {
        if (split) gemm_fp8_kernel<EPI, SPG_FMT_E4M3_ROW, true><<<grid, kThreads, 0, s>>>(g);
        else if (so) gemm_fp8_kernel<EPI, SPG_FMT_E4M3_ROW, false, 4, true><<<grid, kThreads, 0, s>>>(g);
        else gemm_fp8_kernel<EPI, SPG_FMT_E4M3_ROW, false><<<grid, kThreads, 0, s>>>(g);
    } else {
        if (split) gemm_fp8_kernel<EPI, SPG_FMT_E4M3_TENSOR, true><<<grid, kThreads, 0, s>>>(g);
        else if (so) gemm_fp8_kernel<EPI, SPG_FMT_E4M3_TENSOR, false, 4, true><<<grid, kThreads, 0, s>>>(g);
        else gemm_fp8_kernel<EPI, SPG_FMT_E4M3_TENSOR, false><<<grid, kThreads, 0, s>>>(g);
    }
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && g.split_k > 1) e = launch_splitk_reduce(g, p.tiles, s);
    return e;
}

}  // namespace

hipError_t launch_gemm_fp8_half(const GemmArgs &g, hipStream_t s)
{
    switch (g.epilogue) {
    case SPG_EPI_STORE: return launch_half<SPG_EPI_STORE>(g, s);
    case SPG_EPI_ADD: return launch_half<SPG_EPI_ADD>(g, s);
    default: return launch_half<SPG_EPI_SWIGLU>(g, s);
    }
}

hipError_t launch_gemm_fp8(const GemmArgs &g, const spg_plan &p, hipStream_t s)
{
    switch (g.epilogue) {
    case SPG_EPI_STORE: return launch_epi<SPG_EPI_STORE>(g, p, s);
    case SPG_EPI_ADD: return launch_epi<SPG_EPI_ADD>(g, p, s);
    default: return launch_epi<SPG_EPI_SWIGLU>(g, p, s);
    }
}

}  // namespace spg
