// Decode-width GEMM: products of at most 32 tokens, FP8 E4M3 (row or tensor
// scales) and NVFP4, with the same fused epilogues as the tiled kernels.
//
// ninfer PR #160 gives few-token products routes of their own (a small-T
// route and a GEMV for decode widths, reading the same row-major scale
// buffer as the tiled route).  At these widths a product is a stream over
// the weight matrix: the MFMA work per weight byte is 2T flops, far below
// what the matrix cores sustain, so the kernel is shaped for HBM, not MFMA.
//
// Design for CDNA4:
//  * One workgroup per 32 output columns (SWIGLU: 16 columns, i.e. 16 gate
//    rows and their 16 up rows) of one batch entry: 5120 columns give 160
//    workgroups, the 17408-column SwiGLU 1088 (the tiled kernels' 256-column
//    tiles gave 20 and 136 and needed a K split with a second reduction
//    launch).
//  * Its four waves take contiguous quarters of K.  Each wave copies its
//    chunks (128 code bytes of every weight and token row) straight into a
//    private LDS ring with buffer loads to LDS, a few chunks ahead, reads
//    its fragments from there and multiplies with
//    v_mfma_f32_16x16x128_f8f6f4 (FP8) or, after the exact f16 decode of the
//    tiled NVFP4 kernel, v_mfma_f32_16x16x32_f16.  The tokens (at most 32
//    rows) come from L2 with every chunk; each token fragment serves the
//    workgroup's two 16-row weight blocks (SWIGLU: the gate and the up
//    block), two MFMAs per token fragment either way.
//  * K placement: lane l holds row l % 16 and the 32 code bytes at
//    32 (l / 16) of each 128-byte chunk.  For FP8 that is the MFMA's own
//    K order; for NVFP4 the eight k-steps of a chunk take, in lane group
//    l / 16, the K-elements 64 (l / 16) + 8 s + [0, 8) (s = 0..7), the same
//    placement for both operands, so the dot product is unchanged and one
//    NVFP4 block (16 elements) serves a lane for two k-steps.
//  * The four quarters are summed through LDS in a fixed order (0, 1, 2, 3:
//    the result is the same on every run) and one thread per output row
//    fragment applies the scales and the epilogue: 4 adjacent output columns
//    of one token per thread, one 8-byte store.
//  * A wave's chunk range is padded up to a multiple of the ring depth with
//    copies past the range, which read zero through the buffer range check
//    (no memory traffic) and add zero products.
#include "spg_gemm_common.h"

namespace spg {

namespace {

using namespace gemm;

constexpr int kWaves = 4;                 // waves per workgroup, one K quarter each
constexpr int kNarrowThreads = 64 * kWaves;
constexpr int kChunk = 128;               // code bytes of a row per step
// Ring bytes per wave: at most 64 KiB per workgroup, so two or three
// workgroups share a compute unit (measured on the 16-token linears: 16 KiB
// beat 20 KiB by 2-4%, 24 KiB - one SwiGLU workgroup per compute unit - lost
// 25%; eight waves per workgroup instead of four lost 3%).
constexpr int kWaveLds = 16384;

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ v8i cat8(const uint4 &lo, const uint4 &hi)
{
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// Eight E2M1 codes (one 32-bit word, even elements in the low nibbles) ->
// eight f16 values e2m1(c) * S * 2^-7, s2 = (S, S): the conversion applies
// the exact power of two 2^-7 and the packed multiply the block scale (exact:
// at most 6 significant bits, 2^-17 .. 21).
__device__ __forceinline__ v8h decode8(uint32_t w, h2 s2)
{
    const h2 r0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 0.0078125f, 0) * s2;
    const h2 r1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 0.0078125f, 1) * s2;
    const h2 r2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 0.0078125f, 2) * s2;
    const h2 r3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 0.0078125f, 3) * s2;
    return v8h{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
}

// An E4M3 block-scale byte as an f16 pair (exact: E4M3 values 2^-9 .. 448
// are f16 normals with at most 4 significant bits).
__device__ __forceinline__ h2 bscale2(uint32_t code)
{
    const _Float16 h = (_Float16)decode_e4m3(code);
    return h2{h, h};
}

// One chunk of one wave in registers: per lane the code bytes of the
// weight rows (NB blocks) and token rows (TB blocks of 16), and for NVFP4
// their four block-scale bytes.
template <int NB, int TB, bool FP4>
struct Chunk {
    uint4 w[NB][2];
    uint4 a[TB][2];
    uint32_t ws[FP4 ? NB : 1];
    uint32_t as[FP4 ? TB : 1];
};

// EPI: epilogue; FP4: NVFP4 operands (else E4M3); TB: 16-token blocks (1 or
// 2); RB: 16-column blocks per workgroup (each token fragment serves RB
// weight blocks).  Weight block nb = h RB + rb holds rows
// h N/2 + j0 + 16 rb + [0, 16) (h = 1: the up rows of SWIGLU).
//
// Each wave copies its chunks straight into a private LDS ring (buffer
// loads with the LDS bit, as the tiled kernels do): eight lanes fetch one
// whole 128-byte row segment, so a copy instruction moves 8 whole lines
// (fragment-order loads into registers would touch 16 half lines per
// instruction: measured 1.5x slower on the same stream).  A slot holds the
// chunk's weight rows then token rows, 128 bytes each, 16-byte piece j of
// row R at j ^ ((R >> 1) & 7) (the tiled kernels' swizzle: a fragment read
// of 16 rows touches every bank once), then for NVFP4 one 4-byte scale
// word per lane and block, fetched by the lane that reads it.  DEPTH slots
// per wave (at most 16 KiB, at least two slots), so two or three
// workgroups share a compute unit.
template <int EPI, bool FP4, int TB, int RB>
__global__ __launch_bounds__(kNarrowThreads) void gemm_narrow_kernel(const GemmArgs g)
{
    constexpr int NB = (EPI == SPG_EPI_SWIGLU ? 2 : 1) * RB;
    constexpr int kCols = 16 * RB;
    constexpr int ROWS = 16 * (NB + TB);
    constexpr int SLOT = ROWS * kChunk + (FP4 ? (NB + TB) * 256 : 0);
    constexpr int DEPTH = kWaveLds / SLOT < 2 ? 2 : kWaveLds / SLOT > 8 ? 8 : kWaveLds / SLOT;
    // copy instructions per chunk: two per 16 rows, one per scale word set
    constexpr int IPC = 2 * (NB + TB) + (FP4 ? NB + TB : 0);
    static_assert((DEPTH - 1) * IPC <= 63, "vmcnt range");
    // the ring, and after the main loop the four waves' partial sums
    constexpr int kRingBytes = kWaves * DEPTH * SLOT;
    constexpr int kRedBytes = kWaves * NB * TB * 64 * 4 * 4;
    static_assert(kRedBytes <= kRingBytes, "the partial sums fit in the ring");
    __shared__ __attribute__((aligned(2048))) uint8_t lds[kRingBytes];
    auto ring = reinterpret_cast<uint8_t (*)[DEPTH][SLOT]>(lds);
    auto red = reinterpret_cast<float (*)[NB * TB][64 * 4]>(lds);

    clock_mark(g.clocks, 0);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t ncb = g.tiles_n;                       // column blocks (16 RB) per product
    const int64_t b = (int64_t)blockIdx.x / ncb;
    const int64_t j0 = ((int64_t)blockIdx.x - b * ncb) * kCols;
    const int64_t nout = EPI == SPG_EPI_SWIGLU ? g.N / 2 : g.N;
    const int r = lane & 15, kq = lane >> 4;

    // code bytes per row and this wave's chunk range
    const int64_t kbytes = FP4 ? g.K / 2 : g.K;
    const int nch = (int)((kbytes + kChunk - 1) / kChunk);
    const int per = (nch + kWaves - 1) / kWaves;
    const int c_begin = min(nch, wave * per), c_end = min(nch, c_begin + per);

    // copy lanes: lane L fetches row 8 i + L / 8 of a 16-row block (i = 0, 1),
    // global 16-byte piece gj, landing at LDS piece L % 8
    const int crow = lane >> 3, cj = lane & 7;
    uint32_t gj[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) gj[i] = (uint32_t)(cj ^ ((4 * i + (crow >> 1)) & 7));

    // weight rows of block nb: first row wrow0(nb), brows(nb) of them valid
    const int64_t rows = min((int64_t)kCols, nout - j0);
    auto wrow0 = [&](int nb) -> int64_t { return (nb >= RB ? g.N / 2 : 0) + j0 + 16 * (nb % RB); };
    auto brows = [&](int nb) -> int64_t { return max((int64_t)0, min((int64_t)16, rows - 16 * (nb % RB))); };
    const uint8_t *wbase = g.W + (g.stride_w ? b * g.stride_w : 0);
    v4i rw[NB];
    uint32_t woff[NB][2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        rw[nb] = make_rsrc(wbase + wrow0(nb) * g.ldw, (uint32_t)(brows(nb) * g.ldw));
#pragma unroll
        for (int i = 0; i < 2; ++i)
            woff[nb][i] = 8 * i + crow < brows(nb) ? (uint32_t)(8 * i + crow) * (uint32_t)g.ldw + 16 * gj[i] : kOOB;
    }

    // token rows 16 t + 8 i + L / 8
    const uint8_t *abase = g.A + (g.stride_a ? b * g.stride_a : 0);
    const v4i ra = make_rsrc(abase, (uint32_t)(g.M * g.lda));
    uint32_t aoff[TB][2];
#pragma unroll
    for (int t = 0; t < TB; ++t)
#pragma unroll
        for (int i = 0; i < 2; ++i)
            aoff[t][i] = 16 * t + 8 * i + crow < g.M ? (uint32_t)(16 * t + 8 * i + crow) * (uint32_t)g.lda + 16 * gj[i]
                                                     : kOOB;

    // NVFP4 block scales (groups of 16 K-elements, G per row; G % 4 == 0):
    // lane (r, kq) fetches the word of its own row r and groups
    // 16 c + 4 kq .. + 3 of chunk c
    const int64_t G = g.K / 16;
    const bool blocked = FP4 && g.scale_layout == SPG_SCALES_BLOCKED;
    v4i rsw[NB], rsa;
    uint32_t swoff[NB], saoff[TB];
    if constexpr (FP4) {
        if (blocked) {
            // whole planes: 4 KiB per (256-row tile, 256-element stage)
            const int64_t stages = g.K / 256;
            rsa = make_rsrc(g.sa, (uint32_t)(((g.M + 255) / 256) * stages * 4096));
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                rsw[nb] = make_rsrc(g.sw, (uint32_t)(((g.N + 255) / 256) * stages * 4096));
                const int64_t row = wrow0(nb) + r;
                swoff[nb] = r < brows(nb) ? (uint32_t)(((row >> 8) * stages) * 4096 + (row & 255) * 16 + kq * 4)
                                          : kOOB;
            }
#pragma unroll
            for (int t = 0; t < TB; ++t) {
                const int64_t row = t * 16 + r;
                saoff[t] = row < g.M ? (uint32_t)((row & 255) * 16 + kq * 4) : kOOB;
            }
        } else {
            rsa = make_rsrc(g.sa, (uint32_t)(g.M * G));
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                rsw[nb] = make_rsrc((const uint8_t *)g.sw + wrow0(nb) * G, (uint32_t)(brows(nb) * G));
                swoff[nb] = r < brows(nb) ? (uint32_t)(r * G + kq * 4) : kOOB;
            }
#pragma unroll
            for (int t = 0; t < TB; ++t) saoff[t] = t * 16 + r < g.M ? (uint32_t)((t * 16 + r) * G + kq * 4) : kOOB;
        }
    }

    auto slot_addr = [&](int s) -> uint32_t {
        return (uint32_t)__builtin_amdgcn_readfirstlane(
            (int)(uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)&ring[wave][s][0]);
    };

    // copies of chunk c into slot s (chunks past the wave's range, and
    // pieces past K, read as zero: no memory traffic)
    auto issue = [&](int s, int c) {
        const uint32_t base = slot_addr(s);
        const bool live = c < c_end;
        const uint32_t soff = live ? (uint32_t)c * kChunk : 0u;
        const bool kin = live && (int64_t)c * kChunk + 16 * gj[0] < kbytes;
        const bool kin1 = live && (int64_t)c * kChunk + 16 * gj[1] < kbytes;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            dma16(base + (uint32_t)(nb * 16) * kChunk, kin ? woff[nb][0] : kOOB, rw[nb], soff);
            dma16(base + (uint32_t)(nb * 16 + 8) * kChunk, kin1 ? woff[nb][1] : kOOB, rw[nb], soff);
        }
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            dma16(base + (uint32_t)((NB + t) * 16) * kChunk, kin ? aoff[t][0] : kOOB, ra, soff);
            dma16(base + (uint32_t)((NB + t) * 16 + 8) * kChunk, kin1 ? aoff[t][1] : kOOB, ra, soff);
        }
        if constexpr (FP4) {
            const bool gin = live && (int64_t)c * 16 + kq * 4 < G;
            const uint32_t ss = live ? (uint32_t)c * (blocked ? 4096u : 16u) : 0u;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                dma4(base + ROWS * kChunk + nb * 256, gin ? swoff[nb] : kOOB, rsw[nb], ss);
#pragma unroll
            for (int t = 0; t < TB; ++t)
                dma4(base + ROWS * kChunk + (NB + t) * 256, gin ? saoff[t] : kOOB, rsa, ss);
        }
    };

    // fragment reads of slot s: lane (r, kq) takes the 32 bytes 32 kq .. of
    // row r of each block, and its scale words
    const uint32_t fsw = (uint32_t)((r >> 1) & 7);
    const uint32_t fo0 = (uint32_t)r * kChunk + ((((uint32_t)kq * 2) ^ fsw) << 4);
    const uint32_t fo1 = (uint32_t)r * kChunk + ((((uint32_t)kq * 2 + 1) ^ fsw) << 4);
    using C = Chunk<NB, TB, FP4>;
    auto read = [&](C &x, int s) {
        const uint8_t *sl = &ring[wave][s][0];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            x.w[nb][0] = *reinterpret_cast<const uint4 *>(sl + nb * 16 * kChunk + fo0);
            x.w[nb][1] = *reinterpret_cast<const uint4 *>(sl + nb * 16 * kChunk + fo1);
        }
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            x.a[t][0] = *reinterpret_cast<const uint4 *>(sl + (NB + t) * 16 * kChunk + fo0);
            x.a[t][1] = *reinterpret_cast<const uint4 *>(sl + (NB + t) * 16 * kChunk + fo1);
        }
        if constexpr (FP4) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                x.ws[nb] = *reinterpret_cast<const uint32_t *>(sl + ROWS * kChunk + nb * 256 + lane * 4);
#pragma unroll
            for (int t = 0; t < TB; ++t)
                x.as[t] = *reinterpret_cast<const uint32_t *>(sl + ROWS * kChunk + (NB + t) * 256 + lane * 4);
        }
    };

    v4f acc[NB][TB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int t = 0; t < TB; ++t) acc[nb][t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    auto compute = [&](const C &x) {
        if constexpr (!FP4) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const v8i wv = cat8(x.w[nb][0], x.w[nb][1]);
#pragma unroll
                for (int t = 0; t < TB; ++t) {
                    const v8i av = cat8(x.a[t][0], x.a[t][1]);
                    acc[nb][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wv, av, acc[nb][t], 0, 0, 0, 0,
                                                                                  0, 0);
                }
            }
        } else {
            // k-step s: code word s of the lane's 32 bytes, block scale byte s / 2
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                v8h wv[NB], av[TB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const uint4 &q = x.w[nb][s >> 2];
                    const uint32_t word = (s & 3) == 0 ? q.x : (s & 3) == 1 ? q.y : (s & 3) == 2 ? q.z : q.w;
                    wv[nb] = decode8(word, bscale2((x.ws[nb] >> (8 * (s >> 1))) & 0xFFu));
                }
#pragma unroll
                for (int t = 0; t < TB; ++t) {
                    const uint4 &q = x.a[t][s >> 2];
                    const uint32_t word = (s & 3) == 0 ? q.x : (s & 3) == 1 ? q.y : (s & 3) == 2 ? q.z : q.w;
                    av[t] = decode8(word, bscale2((x.as[t] >> (8 * (s >> 1))) & 0xFFu));
                }
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int t = 0; t < TB; ++t)
                        acc[nb][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wv[nb], av[t], acc[nb][t], 0, 0, 0);
            }
        }
    };

    // the ring: chunk c_begin + i sits in slot i % DEPTH.  Before slot i is
    // read, at most (DEPTH - 1) chunks' copies - the later ones - may be
    // outstanding (copies complete in issue order); before it is refilled,
    // its fragment reads have completed.
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) issue(i, c_begin + i);
    for (int c = c_begin; c < c_end; c += DEPTH) {
#pragma unroll
        for (int i = 0; i < DEPTH; ++i) {
            wait_vmem<(DEPTH - 1) * IPC>();
            C x;
            read(x, i);
            wait_lds();
            compute(x);
            issue(i, c + DEPTH + i);
        }
    }
    wait_vmem<0>();

    // ---- the four K quarters, summed in a fixed order (the partial sums
    // reuse the ring once every wave is done with it)
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int t = 0; t < TB; ++t) *reinterpret_cast<v4f *>(&red[wave][nb * TB + t][lane * 4]) = acc[nb][t];
    __syncthreads();
    // thread group (64 threads) q = rb TB + t: column block rb, token block t
    if (tid >= 64 * TB * RB) return;
    const int q = tid >> 6, t = q % TB, rb = q / TB;
    constexpr int NH = EPI == SPG_EPI_SWIGLU ? 2 : 1;   // gate (and up) values
    v4f v[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
        const int slot = (h * RB + rb) * TB + t;
        v[h] = *reinterpret_cast<const v4f *>(&red[0][slot][lane * 4]);
#pragma unroll
        for (int w = 1; w < kWaves; ++w) v[h] += *reinterpret_cast<const v4f *>(&red[w][slot][lane * 4]);
    }

    // ---- epilogue: lane l, register e hold weight row 4 (l / 16) + e of
    // the block (an output column) and token l % 16 of token block t
    const int64_t m = t * 16 + (lane & 15);
    const int64_t col = j0 + 16 * rb + (lane >> 4) * 4;
    if (m < g.M && col < nout) {
        float sa, sw[NH][4];
        if (FP4) {
            // 2^7 per side undoes the decode's 2^-7 offsets; the two tensor
            // scales stay separate factors (each at most 2^7 * 448^-1 * 6^-1
            // * bf16's maximum, below 1.6e37), so their product - which can
            // pass fp32's range when the output does not - is never formed
            sa = 128.0f * *g.tscale_a;
            const float sv = 128.0f * *g.tscale_w;
#pragma unroll
            for (int h = 0; h < NH; ++h)
#pragma unroll
                for (int e = 0; e < 4; ++e) sw[h][e] = sv;
        } else if (g.format == SPG_FMT_E4M3_ROW) {
            const float *psa = (const float *)g.sa + (g.stride_a ? b * g.M : 0);
            const float *psw = (const float *)g.sw + (g.stride_w ? b * g.N : 0);
            sa = psa[m];
#pragma unroll
            for (int h = 0; h < NH; ++h)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sw[h][e] = col + e < nout ? psw[(h ? g.N / 2 : 0) + col + e] : 0.0f;
        } else {
            sa = ((const float *)g.sa)[g.stride_a ? b : 0];
            const float sv = ((const float *)g.sw)[g.stride_w ? b : 0];
#pragma unroll
            for (int h = 0; h < NH; ++h)
#pragma unroll
                for (int e = 0; e < 4; ++e) sw[h][e] = sv;
        }
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (EPI == SPG_EPI_SWIGLU) {
                const float vg = v[0][e] * sa * sw[0][e];
                const float vu = v[NH - 1][e] * sa * sw[NH - 1][e];
                o[e] = swiglu_f32(vg, vu);
            } else {
                o[e] = v[0][e] * sa * sw[0][e];
            }
        }
        const int nv = (int)min((int64_t)4, nout - col);
        if (EPI == SPG_EPI_ADD) {
            if (g.bias_mode != 0) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (e < nv) o[e] += bias_at(g, b, col + e);
            } else {
                const uint16_t *rrow = g.residual + (g.stride_r ? b * g.stride_r : 0) + m * g.ldr + col;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (e < nv) o[e] += __uint_as_float((uint32_t)rrow[e] << 16);
            }
        }
        const uint2 pk = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
        int64_t ld;
        uint16_t *const dst = g.nseg ? out_at(g, b, m, col, ld)   // a 4-column group never straddles segments
                                     : (uint16_t *)g.out + (g.stride_o ? b * g.stride_o : 0) + m * g.ldo + col;
        (void)ld;
        if (nv == 4 && (((uintptr_t)dst) & 7) == 0) {
            *reinterpret_cast<uint2 *>(dst) = pk;
        } else {
            const uint32_t wd[2] = {pk.x, pk.y};
            for (int e = 0; e < nv; ++e) dst[e] = (uint16_t)(wd[e >> 1] >> (16 * (e & 1)));
        }
    }
    clock_mark(g.clocks, 1);
}

template <int EPI, bool FP4>
hipError_t launch_fmt(const GemmArgs &g, hipStream_t s)
{
    constexpr int RB = narrow_cols(EPI) / 16;
    const dim3 grid((unsigned)(g.batch * g.tiles_n));
    if (g.M <= 16)
        gemm_narrow_kernel<EPI, FP4, 1, RB><<<grid, kNarrowThreads, 0, s>>>(g);
    else
        gemm_narrow_kernel<EPI, FP4, 2, RB><<<grid, kNarrowThreads, 0, s>>>(g);
    return hipGetLastError();
}

template <int EPI>
hipError_t launch_epi(const GemmArgs &g, hipStream_t s)
{
    return g.format == SPG_FMT_NVFP4 ? launch_fmt<EPI, true>(g, s) : launch_fmt<EPI, false>(g, s);
}

}  // namespace

// g.tiles_n: column blocks (narrow_cols) per product; one workgroup per block and batch entry.
hipError_t launch_gemm_narrow(const GemmArgs &g, hipStream_t s)
{
    switch (g.epilogue) {
    case SPG_EPI_ADD: return launch_epi<SPG_EPI_ADD>(g, s);
    case SPG_EPI_SWIGLU: return launch_epi<SPG_EPI_SWIGLU>(g, s);
    default: return launch_epi<SPG_EPI_STORE>(g, s);
    }
}

}  // namespace spg
