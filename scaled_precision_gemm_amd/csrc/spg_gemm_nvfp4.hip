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
// accumulation).  The epilogue undoes each operand's 2^-7 offset together
// with its tensor scale, as two factors (2^7 tA, 2^7 tW).  The dense f16
// MFMA rate is half the FP8 rate, so this path is priced against the
// f16/bf16 roofline.
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

// General path (any K multiple of 32): per-thread register-staged loads, the
// tile decoded to f16 in LDS once per stage.
template <int EPI, bool SO = false>
__global__ __launch_bounds__(kThreads, 1) void gemm_nvfp4_general_kernel(const GemmArgs g)
{
    constexpr int kLdsBytes = 4 * kStageBytes;
    __shared__ __attribute__((aligned(2048))) uint8_t lds[kLdsBytes];
    // [stage][operand] views of the flat array
    auto lds_ab = [&](int st, int op) -> uint8_t * { return &lds[(st * 2 + op) * kStageBytes]; };
    __shared__ __attribute__((aligned(16))) float lds_sa[kBM];
    __shared__ __attribute__((aligned(16))) float lds_sw[kBN];
    __shared__ __attribute__((aligned(16))) float lds_bias[bias_words<EPI>()];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const WorkItem wi = work_item(g);
    const Tile T = tile_from_id<EPI>(g, g.tile_begin + wi.tile);

    const int split = wi.split;
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
        splitk_store(g, T, split, acc);   // the slices are summed by splitk_reduce_kernel
        return;
    }
    epilogue<EPI, 4, false, false, SO>(g, T, acc, lds_sa, lds_sw, lds_bias, &lds[(threadIdx.x >> 6) * 4096]);   // after the barrier above
}

// Decode for the fast path, with the hardware conversions.  Every E4M3
// scale S is exact in f16, and v_cvt_scalef32_pk_f16_fp8 turns two scale
// bytes into an f16 pair; a byte permute first puts the lane's scale byte in
// both bytes of the converted word, giving (S, S).  v_cvt_scalef32_pk_f16_fp4
// applies the power-of-two scale 2^-7 exactly, and one packed f16 multiply by
// (S, S) gives e2m1 * S * 2^-7 with no rounding (at most 6 significant bits,
// a multiple of 2^-17, so exact also where it is an f16 subnormal) - the
// value decode8_f16 builds.  Checked on the GPU against the previous decode
// of this path (scale split into a power of two for the conversion and an
// f16 significand) for every code byte in every byte position, with every
// non-negative scale byte in every byte position of its word.
__device__ __forceinline__ h2 scale_pair(uint32_t word, uint32_t sel)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(__builtin_amdgcn_perm(word, word, sel), 1.0f, false);
}

// Pairs 2 H and 2 H + 1 of decode8_cvt: half of a fragment's decode, so that
// the decode of the next k-step spreads evenly over the MFMAs of this one.
template <int H>
__device__ __forceinline__ uint2 decode4_cvt(uint32_t w, h2 s)
{
    const h2 r0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 0.0078125f, 2 * H) * s;
    const h2 r1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 0.0078125f, 2 * H + 1) * s;
    return make_uint2(__builtin_bit_cast(uint32_t, r0), __builtin_bit_cast(uint32_t, r1));
}

__device__ __forceinline__ uint4 decode8_cvt(uint32_t w, h2 s)
{
    const h2 r0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 0.0078125f, 0) * s;
    const h2 r1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 0.0078125f, 1) * s;
    const h2 r2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 0.0078125f, 2) * s;
    const h2 r3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 0.0078125f, 3) * s;
    return make_uint4(__builtin_bit_cast(uint32_t, r0), __builtin_bit_cast(uint32_t, r1),
                      __builtin_bit_cast(uint32_t, r2), __builtin_bit_cast(uint32_t, r3));
}

// ---------------------------------------------------------------------------
// Fast path (K a multiple of 256): the packed codes and block scales are
// copied straight into LDS and each wave decodes its own fragments in
// registers right before the MFMAs.
//
// A stage is 256 K-elements: per operand 256 rows x 128 code bytes (the same
// 128-byte rows, XOR swizzle and copy pattern as the FP8 kernel) plus 256
// rows x 16 scale bytes.  LDS holds two stages (2 x 72 KiB).
//
// K placement.  The MFMA's 16 K-slots per step are split between the lane
// halves (8 each) and any one-to-one placement of K-elements on slots gives
// the same dot product as long as A and W use the same one.  Lane half h of
// k-step 2c + d (c = 16-byte chunk 0..7 of the stage row, d = 0, 1) takes the
// codes in bytes 8h + 4d .. 8h + 4d + 3 of chunk c, i.e. K-elements
// 32c + 16h + 8d + [0, 8): all inside NVFP4 block 2c + h, so one scale byte
// serves a lane for both k-steps and the lane reads both k-steps' codes with
// one 8-byte LDS read.  With the chunk swizzle, the 64 lanes of such a read
// touch every bank twice (the minimum for 512 bytes).
// ---------------------------------------------------------------------------
constexpr int kBKF = 256;                       // K elements per stage
constexpr int kCodeOp = kBM * 128;              // code bytes per operand per stage: 32 KiB
constexpr int kScaleOp = kBM * 16;              // scale bytes per operand per stage: 4 KiB
constexpr int kSlotF = 2 * (kCodeOp + kScaleOp);   // [A codes][W codes][A scales][W scales]
static_assert(4 * 32768 <= 2 * kSlotF, "the epilogue's staged regions fit in the freed slots");

// AM: A blocks per wave that take part (4 in general).  Products of at most
// 32 (64) tokens have only their first 32 (64) tile rows, so AM = 1 (2)
// leaves out the code reads, decodes and MFMAs of the empty A blocks: a stage
// is then paced by the weights (their copies and decode), as for FP8.
template <int EPI, bool SPLIT, int AM = 4, bool SO = false>
__global__ __launch_bounds__(kThreads, 1) void gemm_nvfp4_kernel(const GemmArgs g)
{
    __shared__ __attribute__((aligned(2048))) uint8_t lds[2 * kSlotF];
    __shared__ __attribute__((aligned(16))) float lds_sa[kBM];
    __shared__ __attribute__((aligned(16))) float lds_sw[kBN];
    __shared__ __attribute__((aligned(16))) float lds_bias[bias_words<EPI>()];
    clock_mark(g.clocks, 0);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const WorkItem wi = work_item(g);
    const Tile T = tile_from_id<EPI>(g, g.tile_begin + wi.tile);
    const int64_t k_begin = (int64_t)wi.split * g.k_chunk;
    const int64_t k_end = min(g.K, k_begin + g.k_chunk);
    const int nk = (int)((k_end - k_begin) / kBKF);       // whole stages (K, k_chunk multiples of 256)
    const int64_t Nh = g.N / 2, G = g.K / 16;            // scale bytes per row

    stage_scales<EPI, SPG_FMT_NVFP4>(g, T, lds_sa, lds_sw);

    // ---- copy setup: codes exactly as the FP8 kernel (128-byte rows) ----------
    const uint32_t rib = lane >> 3, pchunk = lane & 7;
    const uint32_t c_even = pchunk ^ ((lane >> 4) & 7u);
    const uint32_t c_odd = pchunk ^ ((4u + (lane >> 4)) & 7u);
    const int64_t a_rows = min((int64_t)kBM, g.M - T.m0);
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
    const uint8_t *A = g.A, *W = g.W;
    const uint8_t *SA = (const uint8_t *)g.sa, *SW = (const uint8_t *)g.sw;
    const v4i rs_a = make_rsrc(A + T.m0 * g.lda, (uint32_t)(a_rows * g.lda));
    const v4i rs_w = make_rsrc(W + w_first * g.ldw, (uint32_t)(w_rows * g.ldw));
    // Scale planes.  Row-major: tile row r's 16 bytes of a stage at row
    // stride K/16.  Blocked: the 16 bytes of physical row p for stage s at
    // ((p / 256) * (K / 256) + s) * 4096 + (p % 256) * 16, so the 256 rows of
    // a stage are 4 KiB of whole lines.  Rows past the matrix read zero (the
    // range check) or the plane's zero padding; either way their codes are
    // zero.
    const bool blk = g.scale_layout == SPG_SCALES_BLOCKED;
    const uint32_t sblk = (uint32_t)(g.K / 256) * 4096u;          // bytes of one row tile's blocks
    const v4i rs_sa = blk ? make_rsrc(SA, (uint32_t)((g.M + 255) / 256) * sblk)
                          : make_rsrc(SA + T.m0 * G, (uint32_t)(a_rows * G));
    const v4i rs_sw = blk ? make_rsrc(SW, (uint32_t)((g.N + 255) / 256) * sblk)
                          : make_rsrc(SW + w_first * G, (uint32_t)(w_rows * G));
    const uint32_t ra0 = (uint32_t)(wave * 64) + rib, rw0 = (uint32_t)((wave & 1) * 64) + rib;
    const uint32_t va_e = ra0 * (uint32_t)g.lda + c_even * 16u, va_o = ra0 * (uint32_t)g.lda + c_odd * 16u;
    const uint32_t vw_e = rw0 * (uint32_t)g.ldw + c_even * 16u, vw_o = rw0 * (uint32_t)g.ldw + c_odd * 16u;
    // scales: lane L of wave w copies the 16 bytes of tile row 64 w + L
    const uint32_t pra = (uint32_t)T.m0 + (uint32_t)(wave * 64 + lane);                  // physical rows
    const uint32_t prw = (uint32_t)w_first + (uint32_t)((wave & 1) * 64 + lane);
    const uint32_t vsa = blk ? (pra >> 8) * sblk + (pra & 255u) * 16u : (uint32_t)(wave * 64 + lane) * (uint32_t)G;
    const uint32_t vsw = blk ? (prw >> 8) * sblk + (prw & 255u) * 16u : (uint32_t)((wave & 1) * 64 + lane) * (uint32_t)G;
    const uint32_t lds_base =
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)&lds[0];

    // 18 copy instructions per wave per stage: 8 + 8 code blocks, 1 + 1 scale blocks
    auto issue_stage = [&](int kt) {
        const int slot = kt & 1;
        const uint32_t kc = (uint32_t)((k_begin + (int64_t)kt * kBKF) / 2);    // code byte offset
        const uint32_t ks = blk ? (uint32_t)((k_begin + (int64_t)kt * kBKF) / kBKF) * 4096u   // stage block
                                : (uint32_t)((k_begin + (int64_t)kt * kBKF) / 16);             // scale byte offset
        const uint32_t sbase = lds_base + (uint32_t)(slot * kSlotF);
        const uint32_t soff_c = (uint32_t)__builtin_amdgcn_readfirstlane((int)kc);
        const uint32_t soff_s = (uint32_t)__builtin_amdgcn_readfirstlane((int)ks);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t la = (uint32_t)__builtin_amdgcn_readfirstlane((int)(sbase + (uint32_t)(wave * 64 * 128 + i * 8 * 128)));
            dma16(la, ((i & 1) ? va_o : va_e) + (uint32_t)(8 * i) * (uint32_t)g.lda, rs_a, soff_c);
            dma16(la + (uint32_t)kCodeOp, ((i & 1) ? vw_o : vw_e) + (uint32_t)(8 * i) * (uint32_t)g.ldw, rs_w, soff_c);
        }
        const uint32_t ls = (uint32_t)__builtin_amdgcn_readfirstlane((int)(sbase + 2u * kCodeOp + (uint32_t)(wave * 64 * 16)));
        dma16(ls, vsa, rs_sa, soff_s);
        dma16(ls + (uint32_t)kScaleOp, vsw, rs_sw, soff_s);
    };

    // ---- fragment addressing ---------------------------------------------------
    const int l32 = lane & 31, khalf = lane >> 5;
    const uint32_t fx = ((uint32_t)l32 >> 1) & 7u;       // swizzle term of every fragment row
    // v_perm selectors putting scale byte h (even chunks) or 2 + h (odd
    // chunks) of a word in its low two bytes
    const uint32_t sel_even = (uint32_t)khalf * 0x0101u, sel_odd = (2u + (uint32_t)khalf) * 0x0101u;
    uint32_t arow[4], wrow[4];
#pragma unroll
    for (int y = 0; y < 4; ++y) arow[y] = (uint32_t)(wm * 128 + y * 32 + l32);
#pragma unroll
    for (int x = 0; x < 4; ++x) wrow[x] = (uint32_t)(wtile_row0<EPI>(wn, x) + l32);

    Acc acc;
    zero_acc(acc);

    // One stage = 8 chunks x 2 k-steps x 16 MFMAs, in a fixed order with the
    // decode and LDS work of the next k-step slotted between the MFMAs of the
    // current one (one wave per SIMD: the MFMA pipe idles whenever the wave
    // stops to wait for LDS or to decode):
    //   k-step (c, 0): after MFMA j decode half j % 2 of fragment j/2 of
    //                  (c, 1); after MFMA 1 read chunk c + 1's codes; after
    //                  MFMA j (j odd) prepare one block scale of chunk c + 1
    //   k-step (c, 1): after MFMA j decode half j % 2 of fragment j/2 of
    //                  (c + 1, 0)
    // Four VALU instructions follow every MFMA.  (Whole fragments after the
    // even MFMAs only - eight, then none - measured 10.7K cycles per stage
    // against 9.7K: the MFMA waits whenever the instructions between two of
    // them outlast its 32 cycles.)
    // Fragments 0..3 are the A blocks y, 4..7 the W blocks x.
    auto compute = [&](int slot) {
        const uint8_t *base = &lds[slot * kSlotF];
        uint4 sc[8];                                   // the 16 scale bytes of each fragment row
#pragma unroll
        for (int f = 0; f < 8; ++f)
            sc[f] = *reinterpret_cast<const uint4 *>(base + 2 * kCodeOp + (f < 4 ? arow[f] * 16 : kScaleOp + wrow[f - 4] * 16));
        auto read_code = [&](int c, int f) -> uint2 {
            const uint32_t off = (((uint32_t)c ^ fx) << 4) + (uint32_t)khalf * 8;
            return *reinterpret_cast<const uint2 *>(base + (f < 4 ? arow[f] * 128 : kCodeOp + wrow[f - 4] * 128) + off);
        };
        // block 2c + h of the stage: byte 2 (c & 1) + h of word c / 2
        auto scale_of = [&](int c, int f) -> h2 {
            const uint4 &v = sc[f];
            const int wi = c >> 1;
            const uint32_t w = wi == 0 ? v.x : wi == 1 ? v.y : wi == 2 ? v.z : v.w;
            return scale_pair(w, (c & 1) ? sel_odd : sel_even);
        };
        uint2 code[2][8];
        h2 bs[2][8];
        uint4 fr[2][8];                                // decoded fragments of the current / next k-step
        // fragment f takes part unless it is an A block past AM
        auto live = [](int f) { return f >= 4 || f < AM; };
#pragma unroll
        for (int f = 0; f < 8; ++f)
            if (live(f)) code[0][f] = read_code(0, f);
#pragma unroll
        for (int f = 0; f < 8; ++f)
            if (live(f)) bs[0][f] = scale_of(0, f);
#pragma unroll
        for (int f = 0; f < 8; ++f)
            if (live(f)) fr[0][f] = decode8_cvt(code[0][f].x, bs[0][f]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int cb = c & 1, nb = cb ^ 1;
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                const int fc = d, fn = d ^ 1;          // fr index of this k-step / the next
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int y = j >> 2, x = j & 3;
                    if (y < AM)
                        acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, fr[fc][4 + x]),
                                                                         __builtin_bit_cast(v8h, fr[fc][y]), acc[x][y],
                                                                         0, 0, 0);
                    // half h of the next k-step's fragment f after MFMA
                    // 2 f + h: four VALU instructions in every MFMA slot
                    const int f = j >> 1, h = j & 1;
                    auto half_decode = [&](uint32_t w, h2 sv) {
                        if (h == 0) {
                            const uint2 r = decode4_cvt<0>(w, sv);
                            fr[fn][f].x = r.x;
                            fr[fn][f].y = r.y;
                        } else {
                            const uint2 r = decode4_cvt<1>(w, sv);
                            fr[fn][f].z = r.x;
                            fr[fn][f].w = r.y;
                        }
                    };
                    if (d == 0) {
                        if (live(f)) half_decode(code[cb][f].y, bs[cb][f]);
                        if (j == 1 && c + 1 < 8) {
#pragma unroll
                            for (int ff = 0; ff < 8; ++ff)
                                if (live(ff)) code[nb][ff] = read_code(c + 1, ff);
                        }
                        if (h == 1 && c + 1 < 8 && live(f)) bs[nb][f] = scale_of(c + 1, f);
                    } else if (c + 1 < 8) {
                        if (j == 0) wait_lds();
                        if (live(f)) half_decode(code[nb][f].x, bs[nb][f]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    };

    // two stages in flight; stage kt + 2 is copied once every wave has
    // finished reading stage kt's slot
    if (nk > 0) issue_stage(0);
    if (nk > 1) issue_stage(1);
    for (int kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk) wait_vmem<18>();
        else wait_vmem<0>();
        block_barrier();                         // stage kt published
        compute(kt & 1);
        if (kt + 2 < nk) {
            wait_lds();
            block_barrier();                     // slot kt & 1 free
            issue_stage(kt + 2);
        }
    }
    __syncthreads();

    if (SPLIT) {
        splitk_store(g, T, wi.split, acc);       // the slices are summed by splitk_reduce_kernel
        clock_mark(g.clocks, 1);
        return;
    }
    // slots free after the barrier: 32 KiB per wave, one region per pass
    epilogue<EPI, 4, false, true, SO>(g, T, acc, lds_sa, lds_sw, lds_bias, &lds[(threadIdx.x >> 6) * 32768]);
    clock_mark(g.clocks, 1);
}

template <int EPI>
hipError_t launch_epi(const GemmArgs &g, const spg_plan &p, hipStream_t s)
{
    const dim3 grid((unsigned)(p.tiles * g.split_k));    // (tile, slice) work items, see work_item
    // the fast path copies 16-byte pieces of the scale planes: both must be
    // 16-byte aligned (rows are, since K / 16 is then a multiple of 16)
    const bool fast = p.bk == kBKF && (((uintptr_t)g.sa | (uintptr_t)g.sw) & 15) == 0;
    const bool so = g.nseg != 0;
    if (fast) {
        if (g.M <= 32) {
            if (g.split_k > 1) gemm_nvfp4_kernel<EPI, true, 1><<<grid, kThreads, 0, s>>>(g);
            else if (so) gemm_nvfp4_kernel<EPI, false, 1, true><<<grid, kThreads, 0, s>>>(g);
            else gemm_nvfp4_kernel<EPI, false, 1><<<grid, kThreads, 0, s>>>(g);
        } else if (g.M <= 64) {
            if (g.split_k > 1) gemm_nvfp4_kernel<EPI, true, 2><<<grid, kThreads, 0, s>>>(g);
            else if (so) gemm_nvfp4_kernel<EPI, false, 2, true><<<grid, kThreads, 0, s>>>(g);
            else gemm_nvfp4_kernel<EPI, false, 2><<<grid, kThreads, 0, s>>>(g);
        } else {
            if (g.split_k > 1) gemm_nvfp4_kernel<EPI, true><<<grid, kThreads, 0, s>>>(g);
            else if (so) gemm_nvfp4_kernel<EPI, false, 4, true><<<grid, kThreads, 0, s>>>(g);
            else gemm_nvfp4_kernel<EPI, false><<<grid, kThreads, 0, s>>>(g);
        }
    } else if (so) {
        gemm_nvfp4_general_kernel<EPI, true><<<grid, kThreads, 0, s>>>(g);
    } else {
        gemm_nvfp4_general_kernel<EPI><<<grid, kThreads, 0, s>>>(g);
    }
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
