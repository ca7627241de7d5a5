// Exported C ABI (include/spg.h): argument validation, the tile / split-K
// selector and kernel launches.  No allocation.  The only global state is
// the per-device address cache of the static scratch array used by
// quantize_block16_noalloc (written once per device, read-only after).
#include <atomic>
#include <math.h>
#include <string.h>

#include "spg_common.h"

using namespace spg;

namespace {

constexpr int64_t kTile = 256;

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }
bool aligned2(const void *p) { return ((uintptr_t)p & 1u) == 0; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int device_units()
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return 256;
    return cus;
}

int64_t n_out_of(const spg_gemm_desc *d, int epi) { return epi == SPG_EPI_SWIGLU ? d->N / 2 : d->N; }

// Checks that do not need the data pointers.
int validate_desc(const spg_gemm_desc *d, int epi)
{
    if (!d) return SPG_EINVAL;
    if (d->format != SPG_FMT_E4M3_ROW && d->format != SPG_FMT_E4M3_TENSOR && d->format != SPG_FMT_NVFP4)
        return SPG_EINVAL;
    if (epi != SPG_EPI_STORE && epi != SPG_EPI_ADD && epi != SPG_EPI_SWIGLU) return SPG_EINVAL;
    if (d->M < 0 || d->N < 0 || d->K < 0 || d->batch < 1) return SPG_EINVAL;
    if (d->stride_a < 0 || d->stride_w < 0 || d->stride_o < 0 || d->stride_r < 0) return SPG_EINVAL;
    if (epi == SPG_EPI_SWIGLU && (d->N & 1)) return SPG_EINVAL;
    const int64_t nout = n_out_of(d, epi);
    if (d->format == SPG_FMT_NVFP4) {
        if (d->K % 32) return SPG_EINVAL;
        if (d->lda < d->K / 2 || d->ldw < d->K / 2) return SPG_EINVAL;
        if (d->batch != 1) return SPG_EUNSUPPORTED;
        if (d->scale_layout != SPG_SCALES_ROW_MAJOR && d->scale_layout != SPG_SCALES_BLOCKED) return SPG_EINVAL;
        if (d->scale_layout == SPG_SCALES_BLOCKED && (d->K % 256)) return SPG_EINVAL;
        if (d->layout != SPG_LAYOUT_NT) return SPG_EUNSUPPORTED;
    } else {
        if (d->K % 16) return SPG_EINVAL;
        // stored row strides: K for K-contiguous operands, M / N for K-major ones
        const int64_t need_a = (d->layout & SPG_LAYOUT_A_KMAJOR) ? d->M : d->K;
        const int64_t need_w = (d->layout & SPG_LAYOUT_W_KMAJOR) ? d->N : d->K;
        if (d->lda < need_a || d->ldw < need_w) return SPG_EINVAL;
        if (d->scale_layout != SPG_SCALES_ROW_MAJOR) return SPG_EINVAL;   // NVFP4 only
        if (d->layout != SPG_LAYOUT_NT) {
            // the transposed copies are read with row stride K; the
            // transpose runs one 64 x 64 block per workgroup
            if (d->K > (INT64_C(1) << 23)) return SPG_EUNSUPPORTED;
            const int64_t blocks = cdiv(d->K, 64) * (cdiv(d->M, 64) + cdiv(d->N, 64)) * d->batch;
            if (blocks >= (INT64_C(1) << 31)) return SPG_EUNSUPPORTED;
        }
    }
    if (d->layout < 0 || d->layout > (SPG_LAYOUT_A_KMAJOR | SPG_LAYOUT_W_KMAJOR)) return SPG_EINVAL;
    if ((d->lda & 15) || (d->ldw & 15)) return SPG_EINVAL;
    // a 256-row tile of codes must fit the 31-bit range of a buffer resource
    if (d->lda > (INT64_C(1) << 23) || d->ldw > (INT64_C(1) << 23)) return SPG_EUNSUPPORTED;
    if ((d->stride_a & 15) || (d->stride_w & 15)) return SPG_EINVAL;
    if (d->ldo < nout) return SPG_EINVAL;
    // ldr == 0: one row (a bias) added to every token row; a bias scale
    // (E4M3 bias codes) only with such a row
    if (epi == SPG_EPI_ADD && d->ldr != 0 && d->ldr < nout) return SPG_EINVAL;
    if (d->bias_scale && (epi != SPG_EPI_ADD || d->ldr != 0)) return SPG_EINVAL;
    // tile ids are computed in 32-bit arithmetic
    {
        const int64_t tm = cdiv(d->M, kTile), tn = epi == SPG_EPI_SWIGLU ? cdiv(nout, kTile / 2) : cdiv(d->N, kTile);
        if (tm > 0 && tn > 0 && (tm * tn > (INT64_C(1) << 28) || d->batch * tm * tn >= (INT64_C(1) << 31)))
            return SPG_EUNSUPPORTED;
    }
    // the epilogue addresses a 32-row block with 32-bit byte offsets
    if (d->ldo >= (INT64_C(1) << 26) || (epi == SPG_EPI_ADD && d->ldr >= (INT64_C(1) << 26)))
        return SPG_EUNSUPPORTED;
    return SPG_OK;
}

// The split-K factor, when the output tiles fill less than half of the
// compute units or the product has at most 64 tokens (its partial tiles
// then hold only those rows, and it streams its weights: more compute units
// stream more of them at once).  FP8 at up to 64 tokens with at most one
// wave of tiles: the cost model below.  Otherwise the split s <= 8
// (K / s >= 1024) that minimises waves(tiles * s) / s, the wave-quantised
// time of the split work.  (With s <= 8 and K / s >= 1024 no slice is empty.)
int choose_split(int64_t tiles, int64_t M, int64_t K, int units, int bk, bool streaming)
{
    if (tiles * 2 > units && M > 64) return 1;
    if (M <= 64 && streaming && tiles <= units) {
        // Few-token FP8 products stream their weights, and a workgroup's fixed
        // cost (pipeline fill, partial stores, its share of the reduction) is
        // worth about eight 128-deep stages: minimise waves * (slice + 1024)
        // over s <= 8 with slices of at least 1024.  Measured (16 tokens):
        // 34816 x 5120 SwiGLU s = 1, 2, 3, 4, 5, 8, 10 -> 52.0, 58.6, 49.2,
        // 53.8, 52.8, 58.2, 63.8 us (picks 3); 5120 x 17408 add s = 4, 6, 8,
        // 12, 16 -> 39.1, 31.3, 28.1, 25-30, 33 us (picks 8: 12 was no faster
        // on average over three A/B rounds and spread wider).
        int best = 1;
        double best_cost = (double)K + 1024.0;   // unsplit: one wave of tiles
        for (int s = 2; s <= 8; ++s) {
            const int64_t chunk = cdiv(cdiv(K, s), bk) * bk;
            if (K / s < 1024) break;
            if ((int64_t)(s - 1) * chunk >= K) continue;   // a slice would be empty
            const double cost = (double)cdiv(tiles * s, units) * ((double)chunk + 1024.0);
            if (cost < best_cost - 1e-9) {
                best_cost = cost;
                best = s;
            }
        }
        return best;
    }
    int best = 1;
    double best_cost = 1.0;
    for (int s = 2; s <= 8; ++s) {
        if (K / s < 1024) break;
        if ((int64_t)(s - 1) * (cdiv(cdiv(K, s), bk) * bk) >= K) continue;   // a slice would be empty
        const double waves = (double)cdiv(tiles * s, units);
        const double cost = waves / s;
        if (cost < best_cost - 1e-9) {
            best_cost = cost;
            best = s;
        }
    }
    return best;
}

// The route model of ninfer PR #167 ("Routing"): a route's cost is its
// waves (ceil(tiles / (units * per_unit))) times the work one unit carries
// through a wave (per_unit * bm * bn), times one calibrated factor per route.
double route_cost(const spg_route_candidate &c, int64_t M, int64_t N, int64_t batch, int32_t units)
{
    if (c.bm <= 0 || c.bn <= 0 || c.per_unit <= 0 || units <= 0) return INFINITY;
    const int64_t tiles = batch * cdiv(M, c.bm) * cdiv(N, c.bn);
    const int64_t slots = (int64_t)units * c.per_unit;
    return c.factor * (double)cdiv(tiles, slots) * (double)c.per_unit * (double)c.bm * (double)c.bn;
}

// The two FP8 tile geometries, in that model, for MI355X (256 compute units,
// one workgroup each: both kernels use most of the LDS):
//   256 x 256 tiles (persistent kernel), factor 1;
//   128 x 256 tiles (the half-height kernel over a grid of 128-row tiles, one
//   per workgroup), factor 1.24: a round of half tiles takes ~0.62 of a round
//   of full tiles (0.53 - 0.67 over several rounds, 0.56 - 0.80 in single
//   rounds: it copies 3/4 of a full tile's bytes per stage for half the
//   MFMAs).  Measured (half route against full tiles, GPU time per call):
//   288 x 21760 x 4096 29 against 45 us, 352 x 21760 x 4096 with a residual
//   add 37 against 66, 384 x 21760 x 8192 69 against 86, 384 x 43008 x 4096
//   72 against 85, 300 x 43520 x 4096 SwiGLU 66 against 80, 96 - 128 tokens
//   (1 - 168 tile columns, K 512 - 5120) 0.35 - 0.91 of the full tiles'
//   time; and the other way 640 x 26624 x 4096 81 against 75, 200 x 40000 x
//   4096 66 against 52, 2048 x 8192 x 4096 59 against 54, 160 x 65536 x 2048
//   35 against 31, 1536 x 16384 x 4096 89 against 86, 4096 x 34816 x 5120
//   SwiGLU 733 against 552.  The factor puts every one of these on its
//   faster side.  At 33 - 64 tokens the half tiles also beat the full
//   kernel's few-token instantiations (which skip the MFMAs of empty row
//   blocks): 0.79 - 0.88 of their time (48 x 34816 x 1024 SwiGLU 11.9
//   against 14.0 us, 64 x 65536 x 2048 24.0 against 27.6 us); those
//   instantiations keep the products split along K.
constexpr spg_route_candidate kFullTile = {256, 256, 1, 1.0};
constexpr spg_route_candidate kHalfTile = {128, 256, 1, 1.24};

// The decode-width kernel for products of at most 32 tokens (kernel 3): one
// workgroup per narrow_cols() output columns and batch entry, so it needs
// enough columns to spread the weight stream (at least 32 blocks of 16
// columns; below that the tiled route's K split gives more workgroups).  Its buffer ranges are 32-bit: a
// blocked NVFP4 scale plane is addressed whole.  NVFP4 scale words are
// copied 4 bytes at a time: K % 64 == 0 (whole words per row) and, for
// row-major planes, 4-byte aligned planes (checked by the caller, which
// has the pointers: `aligned_scales`).
bool narrow_route(const spg_gemm_desc *d, int64_t nout, bool aligned_scales = true)
{
    if (d->M < 1 || d->M > 32 || d->K <= 0) return false;
    if (d->format == SPG_FMT_NVFP4 && (d->K % 64 != 0 || !aligned_scales)) return false;
    const int64_t blocks = d->batch * cdiv(nout, 16);
    if (blocks < 32 || blocks >= (INT64_C(1) << 31)) return false;
    if (d->format == SPG_FMT_NVFP4 && d->scale_layout == SPG_SCALES_BLOCKED &&
        cdiv(d->N, 256) * (d->K / 256) * 4096 >= (INT64_C(1) << 31))
        return false;
    return true;
}

void make_plan(const spg_gemm_desc *d, int epi, int units, spg_plan *p, bool aligned_scales = true)
{
    memset(p, 0, sizeof(*p));
    const int64_t nout = n_out_of(d, epi);
    if (narrow_route(d, nout, aligned_scales)) {
        p->kernel = 3;
        p->bm = d->M <= 16 ? 16 : 32;
        p->bn = narrow_cols(epi);
        p->bk = d->format == SPG_FMT_NVFP4 ? 256 : 128;
        p->split_k = 1;
        p->tiles = d->batch * cdiv(nout, p->bn);
        p->workgroups = p->tiles;
        p->tail_split = 1;
        p->tail_bm = (int32_t)kTile;
        return;
    }
    p->bm = (int32_t)kTile;
    p->bn = (int32_t)kTile;   // weight rows per tile (SWIGLU: 128 gate + 128 up)
    // K elements per pipeline stage: FP8 128; NVFP4 256 (copied straight into
    // LDS) when K is a multiple of 256, else 64 (general path)
    p->bk = d->format == SPG_FMT_NVFP4 ? (d->K % 256 == 0 ? 256 : 64) : 128;
    const int64_t tiles_m = cdiv(d->M, kTile);
    const int64_t tiles_n = epi == SPG_EPI_SWIGLU ? cdiv(nout, kTile / 2) : cdiv(d->N, kTile);
    p->tiles = tiles_m * tiles_n * d->batch;
    // few-token products (both formats stream their weights) take the
    // weight-streaming split model when NVFP4 runs its fast path
    const bool streaming = d->format != SPG_FMT_NVFP4 || p->bk == 256;
    p->split_k = (p->tiles > 0 && d->K > 0) ? choose_split(p->tiles, d->M, d->K, units, p->bk, streaming) : 1;
    p->kernel = d->format == SPG_FMT_NVFP4 ? 1 : 0;
    p->tail_split = 1;
    p->tail_tiles = 0;
    p->tail_bm = (int32_t)kTile;
    // The tail: when the tiles fill several whole rounds of the compute units
    // plus a partial one, the whole rounds run unsplit and the remaining
    // tiles run in a second launch, so that the last round is short instead
    // of mostly idle, in one of two ways:
    //  - split along K into s slices (partial tiles through the workspace
    //    and a reduction), or
    //  - (FP8, at most half a round left) as two 128 x 256 half-height tiles
    //    each, no partials.
    // Each option's time for the last round is estimated from the per-unit
    // rate these kernels reach (FP8 ~9.6, NVFP4 ~4.1 TFLOP/s per compute
    // unit): a K split costs t_tile / s plus the partial tiles' traffic
    // (written and read back at ~4 TB/s) and ~10 us of launches; a half tile
    // ~0.55 t_tile (it carries the same copies per stage for half the MFMAs)
    // plus ~5 us for its launch.  The cheapest of these and the unsplit round
    // (t_tile) is taken.
    if (p->split_k == 1 && p->tiles > units && d->K > 0) {
        const int64_t rem = p->tiles % units;
        if (rem > 0) {
            const double rate = d->format == SPG_FMT_NVFP4 ? 4.1e12 : 9.6e12;
            const double t_tile = 2.0 * kTile * kTile * (double)d->K / rate;
            double best = t_tile;
            int s = (int)(units / rem < 8 ? units / rem : 8);
            while (s > 1 && (d->K / s < 1024 || cdiv(d->K, s) < 2 * (int64_t)p->bk)) --s;
            if (s >= 2) {
                const double t = t_tile / s + 2.0 * (double)rem * s * kTile * kTile * 4.0 / 4e12 + 10e-6;
                if (t < best) {
                    best = t;
                    p->tail_tiles = rem;
                    p->tail_split = s;
                }
            }
            if (p->kernel == 0 && 2 * rem <= units && cdiv(d->K, p->bk) >= 2) {
                const double t = 0.55 * t_tile + 5e-6;
                if (t < best) {
                    best = t;
                    p->tail_tiles = rem;
                    p->tail_split = 1;
                    p->tail_bm = (int32_t)(kTile / 2);
                }
            }
        }
    }
    // Geometry (FP8, unsplit): the full route's cost in the PR #167 model, its
    // partial last round replaced by the tail chosen above, against the
    // half-height kernel over a grid of 128-row tiles.
    if (p->kernel == 0 && p->split_k == 1 && d->K > 0 && p->tiles > 0) {
        const int64_t Nw = tiles_n * kTile;   // tile columns in W rows (SWIGLU: 128 gate + 128 up each)
        double full = route_cost(kFullTile, d->M, Nw, d->batch, units);
        if (p->tail_tiles > 0) {
            const double rate = 9.6e12, t_tile = 2.0 * kTile * kTile * (double)d->K / rate;
            const double tail = p->tail_bm < kTile ? 0.55 * t_tile + 5e-6
                                                   : t_tile / p->tail_split + 2.0 * (double)p->tail_tiles *
                                                     p->tail_split * kTile * kTile * 4.0 / 4e12 + 10e-6;
            full += (tail / t_tile - 1.0) * kFullTile.bm * kFullTile.bn;
        }
        const double half = route_cost(kHalfTile, d->M, Nw, d->batch, units);
        if (half < full) {
            p->kernel = 2;
            p->bm = (int32_t)(kTile / 2);
            p->tiles = d->batch * cdiv(d->M, kTile / 2) * tiles_n;
            p->tail_tiles = 0;
            p->tail_split = 1;
            p->tail_bm = (int32_t)kTile;
            p->workgroups = p->tiles;         // one workgroup per 128-row tile
            return;
        }
    }
    const int64_t main_tiles = p->tiles - p->tail_tiles;
    // The FP8 kernel runs unsplit products with two or more K stages
    // persistently: one workgroup per compute unit walking its tiles.
    if (p->kernel == 0 && p->split_k == 1 && cdiv(d->K, p->bk) >= 2)
        p->workgroups = main_tiles < units ? main_tiles : units;
    else
        p->workgroups = main_tiles * p->split_k;
}

constexpr size_t kWsAlign = 256;
size_t align_ws(size_t b) { return (b + kWsAlign - 1) / kWsAlign * kWsAlign; }

// Workspace bytes of the transposed copies of K-major operands (A first,
// then W, each 256-byte aligned); `a_bytes` gets the A part.
size_t transpose_bytes(const spg_gemm_desc *d, size_t *a_bytes)
{
    size_t a = 0, w = 0;
    if (d->layout & SPG_LAYOUT_A_KMAJOR)
        a = align_ws((size_t)(d->stride_a ? d->batch : 1) * (size_t)d->M * (size_t)d->K);
    if (d->layout & SPG_LAYOUT_W_KMAJOR)
        w = align_ws((size_t)(d->stride_w ? d->batch : 1) * (size_t)d->N * (size_t)d->K);
    if (a_bytes) *a_bytes = a;
    return a + w;
}

size_t plan_workspace(const spg_plan *p)
{
    if (p->split_k > 1) return (size_t)p->tiles * p->split_k * kTile * kTile * sizeof(float);
    if (p->tail_split > 1) return (size_t)p->tail_tiles * p->tail_split * kTile * kTile * sizeof(float);
    return 0;
}

}  // namespace

// ---------------------------------------------------------------------------

SPG_EXPORT const char *spg_status_string(int status)
{
    switch (status) {
    case SPG_OK: return "success";
    case SPG_EINVAL: return "invalid argument";
    case SPG_EUNSUPPORTED: return "unsupported request";
    case SPG_EWORKSPACE: return "workspace missing or too small";
    case SPG_EHIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

SPG_EXPORT void spg_gemm_desc_init(spg_gemm_desc *d, int64_t M, int64_t N, int64_t K, int32_t format)
{
    if (!d) return;
    memset(d, 0, sizeof(*d));
    d->M = M;
    d->N = N;
    d->K = K;
    d->batch = 1;
    d->format = format;
    d->lda = d->ldw = format == SPG_FMT_NVFP4 ? K / 2 : K;
    d->ldo = N;
    d->ldr = N;
}

SPG_EXPORT double spg_route_cost(const spg_route_candidate *c, int64_t M, int64_t N, int64_t batch, int32_t units)
{
    return c ? route_cost(*c, M, N, batch, units) : INFINITY;
}

SPG_EXPORT int spg_route_select(const spg_route_candidate *c, int32_t n, int64_t M, int64_t N, int64_t batch,
                                int32_t units)
{
    if (!c || n <= 0) return -1;
    int best = 0;
    double best_cost = spg_route_cost(&c[0], M, N, batch, units);
    for (int i = 1; i < n; ++i) {
        const double cost = spg_route_cost(&c[i], M, N, batch, units);
        if (cost < best_cost) {
            best_cost = cost;
            best = i;
        }
    }
    return best;
}

SPG_EXPORT int spg_gemm_plan(const spg_gemm_desc *d, int epilogue, int32_t units, spg_plan *plan)
{
    if (!plan) return SPG_EINVAL;
    const int v = validate_desc(d, epilogue);
    if (v != SPG_OK) return v;
    make_plan(d, epilogue, units > 0 ? units : 256, plan);
    return SPG_OK;
}

SPG_EXPORT size_t gemm_scaled_workspace_bytes(const spg_gemm_desc *d, int epilogue)
{
    if (validate_desc(d, epilogue) != SPG_OK) return 0;
    // enough for either plan of a call: the scale planes' alignment (known
    // only at the call) can take an NVFP4 product off the decode-width route
    spg_plan p, q;
    make_plan(d, epilogue, device_units(), &p, true);
    make_plan(d, epilogue, device_units(), &q, false);
    const size_t w = plan_workspace(&p) > plan_workspace(&q) ? plan_workspace(&p) : plan_workspace(&q);
    return transpose_bytes(d, nullptr) + w;
}

// A bf16 output region [o0, o1): one matrix (or segment) of a call.
struct Extent {
    uintptr_t o0, o1;
};

// Checks of an output split (spg_out_split) against the call's shape; its
// segments' extents go to ext[0 .. count).
int validate_split(const spg_out_split *sp, const spg_gemm_desc *d, int64_t nout, Extent *ext)
{
    if (sp->count < 1 || sp->count > SPG_MAX_OUT_SPLITS) return SPG_EINVAL;
    int64_t begin = 0;
    for (int s = 0; s < sp->count; ++s) {
        const int64_t end = sp->col_end[s], width = end - begin, ldo = sp->ldo[s], st = sp->stride_o[s];
        if (width <= 0) return SPG_EINVAL;
        if (s + 1 < sp->count ? (end % 64) != 0 : end != nout) return SPG_EINVAL;
        if (s + 1 < sp->count && end / 64 > 0xFFFF) return SPG_EUNSUPPORTED;   // boundaries held in 16 bits
        if (!sp->out[s] || !aligned16(sp->out[s]) || ldo < width || (ldo & 7) || st < 0) return SPG_EINVAL;
        if (ldo >= (INT64_C(1) << 26)) return SPG_EUNSUPPORTED;
        if (d->batch > 1 && st < (d->M - 1) * ldo + width) return SPG_EINVAL;
        const uintptr_t o0 = (uintptr_t)sp->out[s];
        ext[s] = Extent{o0, o0 + 2 * (uintptr_t)((d->batch - 1) * st + (d->M - 1) * ldo + width)};
        begin = end;
    }
    for (int s = 0; s < sp->count; ++s)
        for (int t = s + 1; t < sp->count; ++t)
            if (ext[s].o0 < ext[t].o1 && ext[t].o0 < ext[s].o1) return SPG_EINVAL;
    return SPG_OK;
}

SPG_EXPORT int gemm_scaled(void *out, const void *A, const void *sa, const void *W, const void *sw,
                           const void *residual, int epilogue, const spg_gemm_desc *d, void *ws,
                           size_t ws_bytes, void *stream)
{
    int v = validate_desc(d, epilogue);
    if (v != SPG_OK) return v;
    const int64_t nout = n_out_of(d, epilogue);
    if (d->M == 0 || nout == 0) return SPG_OK;
    const spg_out_split *split = d->out_split;
    if (!A || !W || !sa || !sw || (split ? out != nullptr : out == nullptr)) return SPG_EINVAL;
    if (!aligned16(A) || !aligned16(W)) return SPG_EINVAL;
    // the output's extents: one matrix, or one per segment
    Extent ext[SPG_MAX_OUT_SPLITS];
    int next = 1;
    if (split) {
        const int v2 = validate_split(split, d, nout, ext);
        if (v2 != SPG_OK) return v2;
        next = split->count;
    } else {
        if (!aligned2(out)) return SPG_EINVAL;
        // batch entries of the output must not overlap (several entries
        // would write the same elements concurrently)
        if (d->batch > 1 && d->stride_o < (d->M - 1) * d->ldo + nout) return SPG_EINVAL;
        ext[0].o0 = (uintptr_t)out;
        ext[0].o1 = ext[0].o0 + 2 * (uintptr_t)((d->batch - 1) * d->stride_o + (d->M - 1) * d->ldo + nout);
    }
    auto overlaps_out = [&](uintptr_t a0, uintptr_t a1) {
        for (int s = 0; s < next; ++s)
            if (a0 < ext[s].o1 && ext[s].o0 < a1) return true;
        return false;
    };
    if (epilogue == SPG_EPI_ADD) {
        const bool codes = d->bias_scale != nullptr;   // E4M3 bias row: 1-byte elements
        if (!residual || (!codes && !aligned2(residual))) return SPG_EINVAL;
        // The residual may be the output itself (read and rewritten by the
        // same lane) only with the same element layout: same pointer, row
        // stride and batch stride.  Any other overlap - including a bias row
        // (ldr == 0) inside the output - is rejected.
        const uintptr_t r0 = (uintptr_t)residual;
        const uintptr_t r1 = r0 + (codes ? 1 : 2) * (uintptr_t)((d->batch - 1) * d->stride_r + (d->M - 1) * d->ldr + nout);
        const bool same = !split && !codes && r0 == ext[0].o0 && d->ldr == d->ldo && d->stride_r == d->stride_o;
        if (overlaps_out(r0, r1) && !same) return SPG_EINVAL;
        if (codes) {
            // read by every workgroup while others write the output
            const uintptr_t b0 = (uintptr_t)d->bias_scale;
            if (!aligned4(d->bias_scale) || overlaps_out(b0, b0 + 4)) return SPG_EINVAL;
        }
    } else if (residual) {
        return SPG_EINVAL;
    }
    if (d->format == SPG_FMT_NVFP4) {
        if (!d->tscale_a || !d->tscale_w || !aligned4(d->tscale_a) || !aligned4(d->tscale_w)) return SPG_EINVAL;
        // blocked planes are read only by the fast path, which copies 16-byte pieces
        if (d->scale_layout == SPG_SCALES_BLOCKED && (!aligned16(sa) || !aligned16(sw))) return SPG_EINVAL;
    } else if (!aligned4(sa) || !aligned4(sw)) {
        return SPG_EINVAL;
    }
    if (((uintptr_t)d->clock_probe & 7u) != 0) return SPG_EINVAL;

    spg_plan p;
    make_plan(d, epilogue, device_units(), &p, aligned4(sa) && aligned4(sw));
    size_t t_a = 0;
    const size_t t_bytes = transpose_bytes(d, &t_a);
    const size_t need = t_bytes + plan_workspace(&p);
    if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws))) return SPG_EWORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    // K-major operands: transposed copies (K contiguous) in the workspace,
    // on the call's stream ahead of the GEMM
    const uint8_t *A_nt = (const uint8_t *)A, *W_nt = (const uint8_t *)W;
    int64_t lda = d->lda, ldw = d->ldw, stride_a = d->stride_a, stride_w = d->stride_w;
    if (d->layout & SPG_LAYOUT_A_KMAJOR) {
        uint8_t *at = (uint8_t *)ws;
        if (launch_transpose_u8(A_nt, d->K, d->M, d->lda, d->stride_a, d->stride_a ? d->batch : 1, at, s) !=
            hipSuccess)
            return SPG_EHIP;
        A_nt = at;
        lda = d->K;
        stride_a = d->stride_a ? d->M * d->K : 0;
    }
    if (d->layout & SPG_LAYOUT_W_KMAJOR) {
        uint8_t *wt = (uint8_t *)ws + t_a;
        if (launch_transpose_u8(W_nt, d->K, d->N, d->ldw, d->stride_w, d->stride_w ? d->batch : 1, wt, s) !=
            hipSuccess)
            return SPG_EHIP;
        W_nt = wt;
        ldw = d->K;
        stride_w = d->stride_w ? d->N * d->K : 0;
    }

    GemmArgs g;
    memset(&g, 0, sizeof(g));
    g.out = out;
    g.A = A_nt;
    g.W = W_nt;
    g.sa = sa;
    g.sw = sw;
    g.residual = (const uint16_t *)residual;
    g.M = d->M;
    g.N = d->N;
    g.K = d->K;
    g.batch = d->batch;
    g.lda = lda;
    g.ldw = ldw;
    g.ldo = d->ldo;
    g.ldr = d->ldr;
    g.stride_a = stride_a;
    g.stride_w = stride_w;
    g.stride_o = d->stride_o;
    g.stride_r = d->stride_r;
    g.sa_bstride = d->M;
    g.sw_bstride = d->N;
    g.format = d->format;
    g.epilogue = epilogue;
    g.tscale_a = d->tscale_a;
    g.tscale_w = d->tscale_w;
    g.scale_layout = d->format == SPG_FMT_NVFP4 ? d->scale_layout : SPG_SCALES_ROW_MAJOR;
    g.bias_mode = epilogue == SPG_EPI_ADD && d->ldr == 0 ? (d->bias_scale ? 2 : 1) : 0;
    g.bias_scale = d->bias_scale;
    if (split) {
        // segment 0 stands for the output in the alignment tests
        g.out = split->out[0];
        g.ldo = split->ldo[0];
        g.stride_o = split->stride_o[0];
        g.nseg = split->count;
        int64_t begin = 0;
        for (int s = 0; s < split->count; ++s) {
            if (s + 1 < split->count)
                g.seg_b[s >> 1] |= (uint32_t)(split->col_end[s] / 64) << (16 * (s & 1));
            g.seg[s].out = (uint16_t *)split->out[s];
            g.seg[s].ldo = split->ldo[s];
            g.seg[s].stride = split->stride_o[s];
            g.seg[s].begin = begin;
            begin = split->col_end[s];
        }
    }
    g.split_k = p.split_k;
    const int64_t unit_k = p.bk;
    g.k_chunk = p.split_k > 1 ? cdiv(cdiv(d->K, p.split_k), unit_k) * unit_k : (d->K > 0 ? d->K : 1);
    g.tiles_m = cdiv(d->M, kTile);
    g.tiles_n = epilogue == SPG_EPI_SWIGLU ? cdiv(nout, kTile / 2) : cdiv(d->N, kTile);
    g.div_per = make_fastdiv((uint32_t)(g.tiles_m * g.tiles_n));
    g.div_span = make_fastdiv((uint32_t)(8 * g.tiles_n));
    g.div_gm_last = make_fastdiv(g.tiles_m % 8 ? (uint32_t)(g.tiles_m % 8) : 8u);
    if (p.split_k > 1) g.partials = (float *)((uint8_t *)ws + t_bytes);
    if (p.kernel == 3) {
        g.tiles_m = 1;
        g.tiles_n = cdiv(nout, narrow_cols(epilogue));
        g.clocks = d->clock_probe;
        return launch_gemm_narrow(g, s) == hipSuccess ? SPG_OK : SPG_EHIP;
    }
    if (p.kernel == 2) {
        // the half-height kernel over a grid of 128-row tiles
        g.tiles_m = cdiv(d->M, kTile / 2);
        g.div_per = make_fastdiv((uint32_t)(g.tiles_m * g.tiles_n));
        g.div_gm_last = make_fastdiv(g.tiles_m % 8 ? (uint32_t)(g.tiles_m % 8) : 8u);
        g.rows128 = 1;
    }
    g.tile_begin = 0;
    g.tile_count = p.tiles - p.tail_tiles;
    auto launch = [&](const GemmArgs &a, const spg_plan &q) {
        return d->format == SPG_FMT_NVFP4 ? launch_gemm_nvfp4(a, q, s) : launch_gemm_fp8(a, q, s);
    };
    spg_plan pm = p;
    pm.tiles = g.tile_count;
    g.clocks = d->clock_probe;
    // the half-height geometry over every tile, or the planned main launch
    hipError_t e = p.kernel == 2 ? launch_gemm_fp8_half(g, s) : launch(g, pm);
    g.clocks = nullptr;                // the clock record covers the main launch only
    if (e == hipSuccess && p.tail_tiles > 0 && p.tail_bm < kTile) {
        // the tail: the last tail_tiles tiles as half-height tiles
        GemmArgs gt = g;
        gt.tile_begin = p.tiles - p.tail_tiles;
        gt.tile_count = p.tail_tiles;
        e = launch_gemm_fp8_half(gt, s);
    } else if (e == hipSuccess && p.tail_tiles > 0) {
        // the tail: the last tail_tiles tiles, split along K, then reduced
        GemmArgs gt = g;
        gt.tile_begin = p.tiles - p.tail_tiles;
        gt.tile_count = p.tail_tiles;
        gt.split_k = p.tail_split;
        gt.k_chunk = cdiv(cdiv(d->K, p.tail_split), unit_k) * unit_k;
        gt.partials = (float *)((uint8_t *)ws + t_bytes);
        spg_plan pt = p;
        pt.tiles = p.tail_tiles;
        pt.split_k = p.tail_split;
        pt.workgroups = p.tail_tiles * p.tail_split;
        e = launch(gt, pt);
    }
    return e == hipSuccess ? SPG_OK : SPG_EHIP;
}

// ---------------------------------------------------------------------------
// quantizers
// ---------------------------------------------------------------------------

SPG_EXPORT int quantize_rowwise(const void *x, int64_t rows, int64_t K, int64_t ldx, uint8_t *q, int64_t ldq,
                                float *scale, void *stream)
{
    if (rows < 0 || K < 0 || (K % 16)) return SPG_EINVAL;
    if (rows == 0 || K == 0) {
        if (rows > 0 && K == 0) return SPG_EINVAL;   // a scale of an empty row is undefined
        return SPG_OK;
    }
    if (!x || !q || !scale) return SPG_EINVAL;
    if (ldx < K || ldq < K || (ldx & 7) || (ldq & 15)) return SPG_EINVAL;
    if (!aligned16(x) || !aligned16(q) || !aligned4(scale)) return SPG_EINVAL;
    hipError_t e = launch_quantize_rowwise((const uint16_t *)x, rows, K, ldx, q, ldq, scale, (hipStream_t)stream);
    return e == hipSuccess ? SPG_OK : SPG_EHIP;
}

SPG_EXPORT size_t quantize_tensor_workspace_bytes(int64_t batch, int64_t rows, int64_t K)
{
    if (batch < 1 || rows < 0 || K < 0) return 0;
    return (size_t)batch * (size_t)amax_parts(rows * K) * sizeof(uint32_t);
}

SPG_EXPORT int quantize_tensor(const void *x, int64_t batch, int64_t rows, int64_t K, int64_t bstride, uint8_t *q,
                               float *scale, void *ws, size_t ws_bytes, void *stream)
{
    if (batch < 1 || rows < 0 || K < 0 || (K % 16)) return SPG_EINVAL;
    if (rows == 0 || K == 0) return SPG_EINVAL;
    if (!x || !q || !scale) return SPG_EINVAL;
    if (bstride < rows * K || (bstride & 7)) return SPG_EINVAL;
    if (!aligned16(x) || !aligned16(q) || !aligned4(scale)) return SPG_EINVAL;
    const size_t need = quantize_tensor_workspace_bytes(batch, rows, K);
    if (!ws || ws_bytes < need || !aligned4(ws)) return SPG_EWORKSPACE;
    hipError_t e = launch_quantize_tensor((const uint16_t *)x, batch, rows, K, bstride, q, scale, (uint32_t *)ws,
                                          amax_parts(rows * K), (hipStream_t)stream);
    return e == hipSuccess ? SPG_OK : SPG_EHIP;
}

SPG_EXPORT size_t quantize_block16_workspace_bytes(int64_t rows, int64_t K)
{
    if (rows < 0 || K < 0) return 0;
    // the single-launch path's sync area, then the two-pass path's partial
    // maxima
    return (size_t)(kBlock16SyncWords + amax_parts(rows * K)) * sizeof(uint32_t);
}

namespace {

// Checks shared by quantize_block16 and quantize_block16_noalloc.
int validate_block16(const void *x, int64_t rows, int64_t K, const uint8_t *q, const uint8_t *bscale,
                     const float *tscale, int layout)
{
    if (rows < 0 || K < 0 || (K % 32)) return SPG_EINVAL;
    if (rows == 0 || K == 0) return SPG_EINVAL;
    if ((layout & ~SPG_QUANT_SINGLE_LAUNCH) != 0 && (layout & ~SPG_QUANT_SINGLE_LAUNCH) != SPG_SCALES_BLOCKED)
        return SPG_EINVAL;
    layout &= ~SPG_QUANT_SINGLE_LAUNCH;
    if (layout == SPG_SCALES_BLOCKED && (K % 256)) return SPG_EINVAL;
    if (!x || !q || !bscale || !tscale) return SPG_EINVAL;
    if (!aligned16(x) || !aligned16(q) || !aligned4(tscale)) return SPG_EINVAL;
    // group indices (padded rows x K/16) are 32-bit in the kernels
    if (((rows + 255) / 256 * 256) * (K / 16) >= (INT64_C(1) << 31)) return SPG_EUNSUPPORTED;
    return SPG_OK;
}

}  // namespace

SPG_EXPORT int quantize_block16_path(int64_t rows, int64_t K)
{
    if (rows <= 0 || K <= 0 || (K % 32)) return -1;
    return quantize_block16_single_launch(rows, K) ? 1 : 2;
}

SPG_EXPORT int quantize_block16(const void *x, int64_t rows, int64_t K, uint8_t *q, uint8_t *bscale, float *tscale,
                                int scale_layout, void *ws, size_t ws_bytes, void *stream)
{
    const int v = validate_block16(x, rows, K, q, bscale, tscale, scale_layout);
    if (v != SPG_OK) return v;
    const size_t need = quantize_block16_workspace_bytes(rows, K);
    if (!ws || ws_bytes < need || !aligned4(ws)) return SPG_EWORKSPACE;
    hipError_t e = launch_quantize_block16((const uint16_t *)x, rows, K, q, bscale, tscale,
                                           scale_layout & ~SPG_QUANT_SINGLE_LAUNCH,
                                           (scale_layout & SPG_QUANT_SINGLE_LAUNCH) != 0, (uint32_t *)ws,
                                           amax_parts(rows * K), (hipStream_t)stream);
    return e == hipSuccess ? SPG_OK : SPG_EHIP;
}

// ---------------------------------------------------------------------------
// quantize_block16_noalloc: quantize_block16 with its scratch in a static
// device array, for callers that cannot allocate (code under graph capture,
// tight serving loops).  The scratch holds the single-launch path's sync
// area (counters, flag and tensor scale, cleared by a small kernel at the
// start of each call, and one maximum per block) and the two-pass path's
// partial maxima: amax_parts() is at most 1024 per tensor, so 10.4 KiB serve
// every size.  Each device holds its
// own copy of the array at its own address, looked up once per device with
// hipGetSymbolAddress; the array's name is never used as an address on the
// host.  Calls on one device share it, so calls that overlap in time on one
// device race.  Every call writes each partial it later reads.
// ---------------------------------------------------------------------------

namespace {

constexpr int64_t kScratchWords = kBlock16SyncWords + 1024;
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) uint32_t scratch[kScratchWords];

namespace {

std::atomic<uintptr_t> g_scratch_ptr[kMaxDevices];

// Address of this device's copy of `scratch` (the current device), or 0 on
// failure.  Concurrent first calls compute the same address: the race is
// benign.
uint32_t *scratch_for_current_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    uintptr_t p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == 0) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
        p = (uintptr_t)ptr;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    return (uint32_t *)p;
}

}  // namespace

SPG_EXPORT int quantize_block16_noalloc(const void *x, int64_t rows, int64_t K, uint8_t *q, uint8_t *bscale,
                                        float *tscale, int scale_layout, void *stream)
{
    const int v = validate_block16(x, rows, K, q, bscale, tscale, scale_layout);
    if (v != SPG_OK) return v;
    const int64_t parts = amax_parts(rows * K);
    if (kBlock16SyncWords + parts > kScratchWords) return SPG_EWORKSPACE;   // beyond the static scratch (not reached today)
    uint32_t *ws = scratch_for_current_device();
    if (!ws) return SPG_EHIP;
    hipError_t e = launch_quantize_block16((const uint16_t *)x, rows, K, q, bscale, tscale,
                                           scale_layout & ~SPG_QUANT_SINGLE_LAUNCH,
                                           (scale_layout & SPG_QUANT_SINGLE_LAUNCH) != 0, ws, parts,
                                           (hipStream_t)stream);
    return e == hipSuccess ? SPG_OK : SPG_EHIP;
}
