/*
 * spg.h - C ABI of the scaled low-precision GEMM path for MI355X (gfx950).
 *
 * The path computes the linear layers of LLM prefill in two primitives, the
 * quantizer and the GEMM - the same split into a quantize primitive and an
 * FP8 GEMM primitive that AstrAI's commit log describes for its API:
 *
 *   1. quantize bf16 activations per token row to FP8 E4M3 (ninfer PR #167,
 *      "The fp8 A8 GEMM stages its operands through TMA", opening summary and
 *      "Measured": row-scaled A8, FP8_E4M3FN weights with row scales), per
 *      matrix (AstrAI's per-tensor E4M3 benchmark on pre-quantized NT operands), or per 16
 *      K-elements to NVFP4 (ninfer PR #160, "The NVFP4 TMA route reads
 *      activation scales as one tile": E2M1 codes, E4M3 scales in tiles of
 *      a block of tokens by 16 groups);
 *   2. multiply by pre-quantized weights with fp32 accumulation and apply the
 *      scales after accumulation, then one fused bf16 epilogue: plain store
 *      (linear), residual add (linear_add) or paired SwiGLU (linear_swiglu)
 *      (PR #167 opening summary, and the maintainer review asking for the
 *      SwiGLU pairing to be handled explicitly).  The output is always bf16,
 *      as AstrAI's commit log fixes it for its GEMM.
 *
 * Conventions for every entry point
 *  - All matrices are row-major.  A is [M, K] (tokens x reduction), W is
 *    [N, K] (weight rows x reduction): both K-contiguous, C = A W^T (the "NT"
 *    layout).
 *  - bf16 tensors are passed as const void* to 16-bit values.
 *  - Every data pointer is a DEVICE pointer owned by the caller; the library
 *    allocates nothing and keeps no mutable global state.  Work is enqueued
 *    on `stream` (a hipStream_t; NULL = the default stream) and is
 *    asynchronous: device faults surface at the caller's next synchronisation.
 *  - Return value: SPG_OK, or an error code.  On any validation error nothing
 *    is enqueued and outputs are untouched.  No C++ exception crosses the ABI.
 *  - Alignment: code and bf16-input pointers and their row strides in bytes
 *    must be multiples of 16 (the kernels load 16-byte vectors); bf16 GEMM
 *    outputs and residuals need only 2-byte alignment, any row stride; fp32
 *    scale pointers 4 bytes.  K must be a multiple of 16 (FP8) or 32 (NVFP4).
 *  - Calls that share a workspace must not overlap in time.
 */
#ifndef SPG_H
#define SPG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
enum {
    SPG_OK = 0,
    SPG_EINVAL = 1,        /* bad argument (null, enum, shape, alignment)   */
    SPG_EUNSUPPORTED = 2,  /* valid request outside what this build runs    */
    SPG_EWORKSPACE = 3,    /* workspace null or smaller than required       */
    SPG_EHIP = 4           /* a HIP call or kernel launch reported an error */
};

/* ---- operand formats (validated, as AstrAI validates its format enum) - */
enum {
    SPG_FMT_E4M3_ROW = 0,    /* E4M3 codes; fp32 scale per row of A and of W  */
    SPG_FMT_E4M3_TENSOR = 1, /* E4M3 codes; one fp32 scale per matrix         */
    SPG_FMT_NVFP4 = 2        /* E2M1 codes 2/byte + E4M3 scale per 16 + fp32  */
};

/* ---- fused epilogues (ninfer: linear, linear_add, linear_swiglu) -------- */
enum {
    SPG_EPI_STORE = 0,   /* out = bf16(v)                                    */
    SPG_EPI_ADD = 1,     /* out = bf16(v + residual)                         */
    SPG_EPI_SWIGLU = 2   /* out[:, j] = bf16(silu(v[:, j]) * v[:, j + N/2])  */
};

/* ---- NVFP4 block-scale plane layouts ---------------------------------- */
enum {
    SPG_SCALES_ROW_MAJOR = 0, /* [rows, K/16], row-major                       */
    SPG_SCALES_BLOCKED = 1,   /* GEMM-native: 4 KiB blocks of 256 rows x 16    */
                              /* scale bytes (one 256-element K stage), blocks */
                              /* ordered by row tile then stage; the last row  */
                              /* tile padded to 256 rows with zero bytes       */
    SPG_QUANT_SINGLE_LAUNCH = 0x100  /* flag for quantize_block16: one launch */
};

const char *spg_status_string(int status);

/* ------------------------------------------------------------------------ */
/* Quantizers                                                               */
/* ------------------------------------------------------------------------ */

/*
 * quantize_rowwise - FP8 E4M3 with one fp32 scale per row (PR #167's
 * row-scaled A8 activations and its row-scaled E4M3FN weights).
 *   For each row r: s_r = fl32(max_k |x_rk| / 448);
 *   q_rk = E4M3 nearest-even of fl32(x_rk / s_r), saturating at +-448, sign of
 *   zero kept; s_r = 0 gives signed-zero codes.
 *   x     : bf16 [rows, K], row stride ldx elements
 *   q     : uint8 codes [rows, K], row stride ldq bytes
 *   scale : fp32 [rows]
 *   K % 16 == 0, ldx >= K, ldq >= K, ldx % 8 == 0, ldq % 16 == 0.
 *   rows == 0 is a no-op; rows > 0 with K == 0 is invalid (no scale exists).
 */
int quantize_rowwise(const void *x, int64_t rows, int64_t K, int64_t ldx,
                     uint8_t *q, int64_t ldq, float *scale, void *stream);

/*
 * quantize_tensor - FP8 E4M3 with one fp32 scale per matrix (AstrAI's
 * per-tensor NT benchmark; a batch of matrices gets one scale each).
 *   x     : bf16, `batch` matrices [rows, K] (row stride K) at x + b*bstride
 *   q     : uint8 codes, matrix b at q + b*rows*K
 *   scale : fp32 [batch], s_b = fl32(amax_b / 448)
 *   ws    : device workspace of at least quantize_tensor_workspace_bytes()
 *   K % 16 == 0, bstride % 8 == 0, bstride >= rows*K.
 */
size_t quantize_tensor_workspace_bytes(int64_t batch, int64_t rows, int64_t K);
int quantize_tensor(const void *x, int64_t batch, int64_t rows, int64_t K, int64_t bstride,
                    uint8_t *q, float *scale, void *ws, size_t ws_bytes, void *stream);

/*
 * quantize_block16 - NVFP4 (PR #160): E2M1 codes, one E4M3 scale per 16
 * consecutive K-elements of a row, one fp32 scale for the tensor.
 *   t     = fl32(amax / 2688)                      (2688 = 448 * 6)
 *   b_g   = E4M3 nearest-even of fl32(amax_g / fl32(6 t)), saturating
 *   e_g   = fl32(dec(b_g) * t)
 *   code  = E2M1 nearest-even of fl32(x / e_g), saturating at +-6; e_g == 0
 *           gives signed zeros
 *   x      : bf16 [rows, K], row stride K
 *   q      : uint8 [rows, K/2]; element k in the low nibble when k is even
 *   bscale : uint8 E4M3 codes.  scale_layout SPG_SCALES_ROW_MAJOR: [rows,
 *            K/16] row-major.  SPG_SCALES_BLOCKED (K % 256 == 0): the plane
 *            PR #160's quantizer writes for its GEMM - the scale of (row r,
 *            group g) at ((r / 256) * (K / 256) + g / 16) * 4096 + (r % 256)
 *            * 16 + g % 16, ceil(rows / 256) * 256 * K / 16 bytes in all,
 *            padding rows zero; the NVFP4 GEMM copies each 4 KiB block with
 *            whole-line loads
 *   tscale : fp32 [1], device
 *   ws     : device workspace of at least quantize_block16_workspace_bytes()
 *            (any contents; the call clears what it uses)
 *   K % 32 == 0.
 * Default: a partial-maximum pass, then an encode pass that reads the
 * tensor again.  scale_layout | SPG_QUANT_SINGLE_LAUNCH requests the single
 * launch (ninfer PR #160's single-launch quantizer, with the tensor amax
 * published by last-block election as AstrAI's commit log publishes its
 * scales): when the tensor fits in the registers of one resident grid,
 * a cooperative launch (after a tiny clearing launch) reads it once, the
 * last block to arrive forms the tensor scale and the others wait for it;
 * otherwise the two passes run.  Results are identical.  Measured on MI355X
 * at 4096 x 6144: two passes 39 us, single launch 70 us (the cooperative
 * launch alone costs ~19 us, and the second read of a cache-resident tensor
 * is cheap), so the single launch pays only where reading the activations
 * twice costs more, e.g. when they do not stay in the last-level cache.
 */
size_t quantize_block16_workspace_bytes(int64_t rows, int64_t K);
/* The path quantize_block16 with SPG_QUANT_SINGLE_LAUNCH takes for [rows, K]
 * on the current device: 1 = single launch, 2 = two passes (the tensor does
 * not fit one resident grid); -1 for an invalid shape.  Host query. */
int quantize_block16_path(int64_t rows, int64_t K);
int quantize_block16(const void *x, int64_t rows, int64_t K, uint8_t *q, uint8_t *bscale,
                     float *tscale, int scale_layout, void *ws, size_t ws_bytes, void *stream);

/*
 * quantize_block16_noalloc - quantize_block16 for callers that cannot
 * allocate: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments and results as quantize_block16
 * without the workspace: its scratch (the partial maxima of the tensor amax,
 * at most 1024 x 4 bytes, and the single-launch path's counters, flag and
 * block maxima, cleared by the call) is a static device array of 10.4 KiB
 * that each GPU
 * the library runs on holds until the process ends.  It calls no allocating
 * routine.  Calls on one GPU share that array: calls that overlap in time on
 * one GPU race (serialize them, e.g. on one stream).  SPG_EWORKSPACE if a
 * size ever needed more partial maxima than the array holds (no size does
 * today), SPG_EHIP if the array's device address cannot be obtained.
 */
int quantize_block16_noalloc(const void *x, int64_t rows, int64_t K, uint8_t *q, uint8_t *bscale,
                             float *tscale, int scale_layout, void *stream);

/* ------------------------------------------------------------------------ */
/* GEMM                                                                      */
/* ------------------------------------------------------------------------ */

/*
 * Operand storage (spg_gemm_desc.layout, flags).  The product is always
 * out = epilogue(scale * A W^T) with A the logical M x K and W the logical
 * N x K matrix; a flag stores that operand with K as its rows instead - the
 * layouts of the backward products (AstrAI commit log, the crosswise
 * backward GEMM entries: dX = dY W reads W K-major, dW = dY^T X reads both
 * operands K-major).  FP8 formats only (NVFP4: SPG_EUNSUPPORTED).
 */
typedef enum {
    SPG_LAYOUT_NT = 0,         /* A [M, K], W [N, K]: K contiguous in both    */
    SPG_LAYOUT_A_KMAJOR = 1,   /* A stored [K, M]: lda >= M (row stride)       */
    SPG_LAYOUT_W_KMAJOR = 2    /* W stored [K, N]: ldw >= N                    */
} spg_layout;

/*
 * Output split along N (split-N epilogue): the output columns of one product
 * go to up to SPG_MAX_OUT_SPLITS separate matrices, one per column range -
 * the fused input projections (q | k | v ...) that ninfer PR #167 lists
 * among the GEMM's call sites (attn_input_proj, gdn_input_proj) computed as
 * one GEMM over the row-concatenated weights.  Segment s holds output
 * columns [col_end[s-1], col_end[s]) (col_end[-1] = 0) as a bf16 matrix with
 * row stride ldo[s] and batch stride stride_o[s] (elements).
 *   count        : 1 .. SPG_MAX_OUT_SPLITS
 *   col_end      : strictly increasing; every end but the last a multiple of
 *                  64; the last equals the output width (N, N/2 for SWIGLU)
 *   out[s]       : device, 16-byte aligned, ldo[s] a multiple of 8 with
 *                  ldo[s] >= the segment's width and < 2^26; with batch > 1,
 *                  stride_o[s] >= (M - 1) * ldo[s] + width
 *   No two segments, and no segment and a residual or bias, may overlap.
 * Anything else: SPG_EINVAL.  The values are those of the unsplit output.
 */
#define SPG_MAX_OUT_SPLITS 8
typedef struct spg_out_split {
    int32_t count;
    int32_t reserved;
    int64_t col_end[SPG_MAX_OUT_SPLITS];
    void *out[SPG_MAX_OUT_SPLITS];
    int64_t ldo[SPG_MAX_OUT_SPLITS];
    int64_t stride_o[SPG_MAX_OUT_SPLITS];
} spg_out_split;

/*
 * Shape and layout of one gemm_scaled call.  Initialise with
 * spg_gemm_desc_init() so unused fields are zero and optional pointers NULL
 * (AstrAI: default-initialised parameter structs never carry garbage).
 *   M, N, K  : A [M, K], W [N, K]; out [M, N], or [M, N/2] for SWIGLU
 *   batch    : number of independent products (>= 1)
 *   lda, ldw : row strides of A and W in bytes of codes (NVFP4: bytes of
 *              packed codes, >= K/2); at most 2^23 (else SPG_EUNSUPPORTED)
 *   ldo, ldr : row strides of out and residual in bf16 elements; below 2^26
 *              (else SPG_EUNSUPPORTED).  ldr == 0 makes the residual one row
 *              of N (N/2 never applies: ADD only) bf16 values added to every
 *              token row: the bf16 bias epilogue (AstrAI commit log for
 *              gemm.cuh, the commit fusing the bias: a raw bf16 bias added in
 *              the epilogue after the operand scales, instead of a separate
 *              elementwise add)
 *   stride_* : batch strides (bytes for A/W codes, elements for out and
 *              residual); 0 broadcasts one matrix to every batch entry
 *              (AstrAI broadcasts batches of one through a zero stride)
 *   format   : SPG_FMT_*
 *   scale_layout : NVFP4 only, the layout of both block-scale planes
 *              (SPG_SCALES_ROW_MAJOR, or SPG_SCALES_BLOCKED with K % 256 == 0)
 *   tscale_a, tscale_w : NVFP4 only, device fp32 [1] tensor scales
 *   clock_probe : optional (NULL by default), device, 4 x uint64.  When
 *              set, thread 0 of the first workgroup of the call's main GEMM
 *              launch stores the shader-clock counter when the kernel
 *              starts and ends (clock_probe[0], [1]) and the 100 MHz
 *              reference counter at the same points ([2], [3]): the shader
 *              clock the kernel ran at is (c1 - c0) / (c3 - c2) * 100 MHz.
 *              A measurement aid only; results do not depend on it.
 *   bias_scale : optional (NULL by default), device, one fp32 value.  When
 *              set, the ADD epilogue's one-row residual (ldr == 0, a bias)
 *              holds E4M3 codes, N bytes per batch entry (stride_r in bytes),
 *              and bias j enters as dec(code_j) * bias_scale, formed in fp32
 *              after the operand scales and before the one rounding to bf16;
 *              one scale serves every batch entry.  NULL keeps the raw bf16
 *              bias row (AstrAI commit log, the commit fusing the bias into
 *              the GEMM epilogue: a null bias scale means a bf16 bias, a
 *              non-null one FP8 storage dequantized in the epilogue).  Set
 *              with any other epilogue or with ldr != 0: SPG_EINVAL.
 *   out_split : optional (NULL by default), host memory read during the
 *              call: the output as column segments (spg_out_split above).
 *              When set, gemm_scaled's `out` must be NULL and ldo, stride_o
 *              are not used.
 *   layout   : SPG_LAYOUT_* flags (0 by default).  A K-major operand is
 *              copied transposed into the workspace by the call (a byte
 *              transpose, HBM-bound) and the product then runs as for
 *              SPG_LAYOUT_NT; lda / ldw are the stored row strides (>= M,
 *              >= N; multiples of 16), stride_a / stride_w the stored batch
 *              strides; sa / sw keep their meaning (per output row / column,
 *              or per tensor).
 */
typedef struct spg_gemm_desc {
    int64_t M, N, K, batch;
    int64_t lda, ldw, ldo, ldr;
    int64_t stride_a, stride_w, stride_o, stride_r;
    int32_t format;
    int32_t scale_layout;
    const float *tscale_a;
    const float *tscale_w;
    uint64_t *clock_probe;
    const float *bias_scale;
    const spg_out_split *out_split;
    int32_t layout;
    int32_t reserved2;
} spg_gemm_desc;

/* Zero every field, set batch = 1 and the dense strides for M, N, K. */
void spg_gemm_desc_init(spg_gemm_desc *d, int64_t M, int64_t N, int64_t K, int32_t format);

/*
 * gemm_scaled - out = epilogue(scale * (A W^T)), fp32 accumulation.
 *   out      : bf16 [M, N] (STORE, ADD) or [M, N/2] (SWIGLU); NULL when
 *              d->out_split gives the output as column segments
 *   A, W     : codes as described by d->format
 *   sa, sw   : E4M3_ROW: fp32 [M] and fp32 [N] (per batch entry: + b*M, b*N
 *              unless that operand's batch stride is 0);
 *              E4M3_TENSOR: fp32 [batch] each (index 0 when broadcast);
 *              NVFP4: E4M3 block-scale planes [M, K/16] and [N, K/16] in
 *              d->scale_layout (NVFP4 requires batch == 1)
 *   residual : bf16 [M, N] (or one row [N] when ldr == 0; E4M3 codes [N]
 *              when d->bias_scale is set), required for SPG_EPI_ADD, NULL
 *              otherwise; it may be the output itself (residual == out,
 *              ldr == ldo, stride_r == stride_o); any other overlap of the
 *              two, a bias row inside the output included, is SPG_EINVAL,
 *              and so is a bias scale inside the output
 *   epilogue : SPG_EPI_*; SWIGLU pairs W rows j (gate) and j + N/2 (up) and
 *              needs N even
 *   ws       : device workspace of at least gemm_scaled_workspace_bytes(d, epilogue)
 *              (may be NULL when that is 0): K-split partial tiles, and the
 *              transposed copies of K-major operands
 *   With batch > 1 the output entries must not overlap:
 *   stride_o >= (M - 1) * ldo + n_out, else SPG_EINVAL.
 * Results: each element within 2^-8 |y| + 2^-12 S of the exact value y,
 * where S is the scaled sum of |products| (fp32 accumulation order is free).
 */
size_t gemm_scaled_workspace_bytes(const spg_gemm_desc *d, int epilogue);
int gemm_scaled(void *out, const void *A, const void *sa, const void *W, const void *sw,
                const void *residual, int epilogue, const spg_gemm_desc *d,
                void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------ */
/* Tile / route selection (host only, no device access)                     */
/* ------------------------------------------------------------------------ */

/*
 * The route model of PR #167 ("Routing"): compare quantised costs, "waves
 * needed times the work one SM carries through a wave", one empirical factor
 * per route.  A candidate is a tile of bm x bn outputs of which per_unit run
 * concurrently on one compute unit, with a cost factor; its cost for an
 * M x N output over `batch` products is
 *     factor * ceil(tiles / (units * per_unit)) * per_unit * bm * bn,
 * tiles = batch * ceil(M/bm) * ceil(N/bn).  spg_route_select returns the
 * index of the cheapest candidate (the first on ties).
 */
typedef struct spg_route_candidate {
    int32_t bm, bn, per_unit;
    double factor;
} spg_route_candidate;

double spg_route_cost(const spg_route_candidate *c, int64_t M, int64_t N, int64_t batch, int32_t units);
int spg_route_select(const spg_route_candidate *c, int32_t n, int64_t M, int64_t N, int64_t batch,
                     int32_t units);

/*
 * The plan gemm_scaled would launch for `d` on a device with `units` compute
 * units: tile shape, K-split, the number of workgroups and the tail (split
 * along K, or run as half-height tiles).  For unsplit FP8 products the tile
 * geometry (256 x 256, or 128 x 256 over the whole
 * product) is chosen with the route model above: factor 1 for 256 x 256,
 * 1.24 for 128 x 256 (measured: a round of half tiles takes ~0.62 of a
 * round of full tiles), the 256 x 256 route's partial last round replaced
 * by its tail.  Products of at most 32 tokens with at least 32
 * blocks of 16 output columns (over the batch) take the decode-width kernel
 * (kernel 3): one workgroup per 32 output columns (SWIGLU: 16), K split
 * between its four waves and summed in LDS, no workspace (ninfer PR #160
 * gives decode widths a GEMV route of their own).
 * Returns SPG_OK or the validation error gemm_scaled would return.  The
 * workspace holds one fp32 256x256 partial tile per split tile and slice.
 */
typedef struct spg_plan {
    int32_t bm, bn, bk;      /* workgroup tile (output rows, weight rows, K)  */
    int32_t split_k;         /* K partitions reduced through the workspace    */
    int64_t tiles;           /* output tiles over the whole batch             */
    int64_t workgroups;      /* workgroups of the first launch: tiles (minus  */
                             /* the tail) * split_k, or at most one per       */
                             /* compute unit when the FP8 kernel runs an      */
                             /* unsplit product persistently                  */
    int32_t kernel;          /* 0: FP8 256 x 256 tiles; 1: NVFP4; 2: FP8      */
                             /* 128 x 256 tiles (bm = 128) over the product,  */
                             /* one workgroup each (tiles counts 128-row      */
                             /* tiles);                                       */
                             /* 3: decode width (both formats; bm = 16 or 32  */
                             /* tokens, bn = 32 output columns, 16 for        */
                             /* SWIGLU; tiles = workgroups =                  */
                             /* batch * ceil(columns / bn))                   */
    int32_t tail_split;      /* > 1: the last tail_tiles tiles run in a second */
                             /* launch split tail_split ways along K (whole   */
                             /* rounds of tiles stay unsplit), else 1         */
    int64_t tail_tiles;
    int32_t tail_bm;         /* output rows per workgroup of the tail launch: */
                             /* 256, or 128 when the tail tiles run unsplit   */
                             /* as two half-height tiles each (FP8 formats)   */
    int32_t reserved;
} spg_plan;

int spg_gemm_plan(const spg_gemm_desc *d, int epilogue, int32_t units, spg_plan *plan);

/* ---- measurement probes (not steps of the method) ------------------------
 * The machine's own ceilings, measured on the device at hand and quoted next
 * to the GEMM figures (ninfer PR #160 compares its kernels with a measured
 * MMA ceiling in the same way).
 *
 * spg_probe_mfma: `workgroups` workgroups of 256 threads each run `iters`
 * rounds of four independent back-to-back MFMAs on register operands (fixed
 * pseudo-random bits, no NaN or infinity): kind 0 = E4M3 32x32x64 (131072
 * flops each), kind 1 = f16 32x32x16 (32768 flops).  Total flops =
 * workgroups * 4 waves * iters * 4 * flops-per-MFMA.  sink: device, one
 * float per thread (workgroups * 256), keeps the results live.  clocks:
 * device, 4 x uint64: shader-clock counter before / after the loop of wave 0
 * of workgroup 0, then the 100 MHz reference counter before / after, so
 * (c[1] - c[0]) / (c[3] - c[2]) * 100 MHz is the shader clock it ran at.
 * SPG_EINVAL for kind not 0/1, iters or workgroups < 1, null or misaligned
 * pointers.
 *
 * spg_probe_read: a read-only stream over `bytes` (a multiple of 16, >= 16)
 * at device pointer src (16-byte aligned) by `workgroups` workgroups of 256
 * threads; thread t writes to sink[t] the XOR of the 32-bit words it read
 * (words t*4 .. t*4+3 of every 16-byte vector v = t, t + 256 * workgroups,
 * ...), so the XOR of all sink words is the XOR of the whole buffer.
 */
int spg_probe_mfma(int kind, int64_t iters, int32_t workgroups, float *sink, uint64_t *clocks, void *stream);

int spg_probe_read(const void *src, int64_t bytes, int32_t workgroups, uint32_t *sink, void *stream);

/*
 * spg_probe_fp4_rounding: the NVFP4 quantizers round quotients to E2M1 with
 * the conversion instruction v_cvt_scalef32_pk_fp4_f32 (scale 1); ninfer PR
 * #160's format needs round-to-nearest-even with saturation at +-6 and the
 * sign of zero kept.  This probe converts every binary32 value that is not a
 * NaN with the instruction and with the library's bit-level E2M1 encoder and
 * counts the differences.  result: device, 34 x uint32 (4-byte aligned),
 * written on `stream`: [0] the number of differences, [1] how many were
 * recorded, then up to 16 pairs (input bits, instruction code | encoder code
 * << 8).  SPG_EINVAL for a null or misaligned result.
 */
int spg_probe_fp4_rounding(uint32_t *result, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SPG_H */
