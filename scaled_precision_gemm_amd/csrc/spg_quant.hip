// Quantizer kernels for gfx950: per-row and per-tensor FP8 E4M3, and the
// NVFP4 block-16 format.
//
// Row-scaled FP8 follows ninfer PR #167 ("The fp8 A8 GEMM stages its operands
// through TMA", opening summary: row-scaled A8; "Measured": E4M3FN weights
// with row scales).  Per-tensor FP8 follows AstrAI's per-tensor NT benchmark,
// whose quantizer reduces an amax before encoding.  NVFP4 follows ninfer PR
// #160 (E2M1 codes, an E4M3 scale per 16 K-elements, an fp32 tensor scale).
//
// All three are HBM-bound streams (2 bytes in, 1 or 0.56 bytes out per
// element), provided the per-element work stays small (see RowScale).  Loads are 16-byte vectors of 8 bf16; amax is taken on the bf16
// bit patterns with the sign cleared (for non-negative floats the unsigned
// integer order is the numeric order), reduced across the wavefront with
// lane shuffles, then across waves through LDS.  Scales and ratios use IEEE
// binary32 division (no fast-math), so the codes are bit-identical to a
// correctly rounded reference.
#include "spg_common.h"

#include <type_traits>

namespace spg {

namespace {

constexpr int kThreads = 256;

// max(|bf16|) over the 8 values of a 16-byte vector, as a bit pattern.
__device__ __forceinline__ uint32_t amax8(const uint4 &v)
{
    uint32_t m = 0;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t lo = w[i] & 0x7FFFu, hi = (w[i] >> 16) & 0x7FFFu;
        m = max(m, max(lo, hi));
    }
    return m;
}

// Division by a row's scale, made cheap.  The E4M3 code of fl32(x / s) is
// needed for every element; s = fl32(amax / 448) is fixed per row (per
// matrix for the per-tensor format).  Instead of an IEEE division per element:
//   xs = x k, ss = s k        (k = 2^100 when amax < 2^-40, else 1: exact)
//   r  = fl32(1 / ss)         (once per row)
//   q0 = fl32(xs r);  e = fma(-q0, ss, xs);  q = copysign(fma(e, r, q0), x)
// then q is clamped to [-448, 448] and converted with v_cvt_pk_fp8_f32
// (E4M3FN, round to nearest even).  q can differ from fl32(x / s) by an ulp
// only where the code cannot change; the scaling keeps the residual e from
// underflowing for tiny rows.  Checked exhaustively on the GPU against IEEE
// division followed by the reference RNE encoder: every positive finite bf16
// amax with every bf16 x, |x| <= amax, gives the same code (and the clamped
// conversion matches the reference encoder for every finite binary32).
// Rows whose scale is zero, infinite or NaN keep the exact slow path.
struct RowScale {
    float s, k, ss, r;
    bool fast;
};

__device__ __forceinline__ RowScale row_scale(float amax)
{
    RowScale t;
    t.s = amax / 448.0f;
    t.fast = t.s > 0.0f && t.s <= 3.40282347e38f;
    t.k = amax < 0x1p-40f ? 0x1p100f : 1.0f;
    t.ss = t.s * t.k;
    t.r = 1.0f / t.ss;
    return t;
}

// SCALED: the row needs the 2^100 scaling (k != 1); the common case skips
// the multiplications by k (exact either way: k = 1 makes them identities).
// The clamp is one v_med3_f32.
template <bool SCALED>
__device__ __forceinline__ float quot(float x, const RowScale &t)
{
    const float xs = SCALED ? x * t.k : x;
    const float q0 = xs * t.r;
    const float e = __builtin_fmaf(-q0, t.ss, xs);
    const float q = __builtin_copysignf(__builtin_fmaf(e, t.r, q0), x);
    return __builtin_amdgcn_fmed3f(q, -448.0f, 448.0f);
}

// Encode 8 bf16 values (one 16-byte vector) to 8 E4M3 codes.  MODE (the
// same for a whole row or matrix): 0 the exact slow path (zero, infinite or
// NaN scale: IEEE division or signed zeros), 1 the fast path, 2 the fast path
// with the 2^100 scaling of tiny rows.
template <int MODE>
__device__ __forceinline__ uint2 encode8_e4m3(const uint4 &v, const RowScale &t)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t out[2];
    if (MODE > 0) {
        constexpr bool SC = MODE == 2;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            int d = __builtin_amdgcn_cvt_pk_fp8_f32(quot<SC>(bf16_lo(w[2 * h]), t), quot<SC>(bf16_hi(w[2 * h]), t),
                                                    0, false);
            d = __builtin_amdgcn_cvt_pk_fp8_f32(quot<SC>(bf16_lo(w[2 * h + 1]), t),
                                                quot<SC>(bf16_hi(w[2 * h + 1]), t), d, true);
            out[h] = (uint32_t)d;
        }
    } else {
        const float s = t.s;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint32_t c0, c1, c2, c3;
            if (s > 0.0f) {
                c0 = encode_e4m3(bf16_lo(w[2 * h]) / s);
                c1 = encode_e4m3(bf16_hi(w[2 * h]) / s);
                c2 = encode_e4m3(bf16_lo(w[2 * h + 1]) / s);
                c3 = encode_e4m3(bf16_hi(w[2 * h + 1]) / s);
            } else {   // zero scale: signed zeros
                c0 = (w[2 * h] >> 8) & 0x80u;
                c1 = (w[2 * h] >> 24) & 0x80u;
                c2 = (w[2 * h + 1] >> 8) & 0x80u;
                c3 = (w[2 * h + 1] >> 24) & 0x80u;
            }
            out[h] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
        }
    }
    return make_uint2(out[0], out[1]);
}

// Calls f(std::integral_constant<int, MODE>) with the encode mode of scale t.
template <typename F>
__device__ __forceinline__ void with_encode_mode(const RowScale &t, F &&f)
{
    if (!t.fast)
        f(std::integral_constant<int, 0>{});
    else if (t.k == 1.0f)
        f(std::integral_constant<int, 1>{});
    else
        f(std::integral_constant<int, 2>{});
}

// Block-wide max of a per-thread value (256 threads = 4 waves).
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t *lds4)
{
    v = wave_max_u32(v);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) lds4[wave] = v;
    __syncthreads();
    uint32_t r = max(max(lds4[0], lds4[1]), max(lds4[2], lds4[3]));
    __syncthreads();
    return r;
}

__device__ __forceinline__ uint4 ld16(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }

// ---------------------------------------------------------------------------
// Row-wise FP8.  TPR threads cooperate on one row (TPR = 64: one wave per
// row, 4 rows per block; TPR = 256: one row per block).  Each thread keeps up
// to CACHE 16-byte vectors of its row in registers between the amax pass and
// the encode pass; CACHE = 0 re-reads the row (served from L2) instead.
// The cached vectors are all loaded before any is used, so a thread has its
// whole share of the row in flight at once.
// ---------------------------------------------------------------------------
template <int TPR, int CACHE>
__global__ __launch_bounds__(kThreads) void quant_rowwise_kernel(
    const uint16_t *__restrict__ x, int64_t rows, int64_t K, int64_t ldx,
    uint8_t *__restrict__ q, int64_t ldq, float *__restrict__ scale)
{
    __shared__ uint32_t lds4[4];
    constexpr int RPB = kThreads / TPR;
    const int lane = threadIdx.x % TPR;
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
    const bool live = row < rows;
    const uint16_t *xr = x + (live ? row : 0) * ldx;
    const int64_t nvec = K / 8;

    uint32_t m = 0;
    uint4 cache[CACHE > 0 ? CACHE : 1];
    if (CACHE > 0) {
#pragma unroll
        for (int c = 0; c < CACHE; ++c) {
            int64_t v = lane + (int64_t)c * TPR;
            if (live && v < nvec) {
                cache[c] = ld16(xr + v * 8);
                m = max(m, amax8(cache[c]));
            }
        }
    } else {
        for (int64_t v = lane; live && v < nvec; v += TPR) m = max(m, amax8(ld16(xr + v * 8)));
    }

    if (TPR == kThreads) {
        m = block_max_u32(m, lds4);
    } else {
#pragma unroll
        for (int off = TPR / 2; off >= 1; off >>= 1) {
            uint32_t o = (uint32_t)__shfl_xor((int)m, off, 64);
            m = max(m, o);
        }
    }
    if (!live) return;
    const RowScale t = row_scale(__uint_as_float(m << 16));
    if (lane == 0) scale[row] = t.s;
    uint8_t *qr = q + row * ldq;
    with_encode_mode(t, [&](auto mode_c) {
        constexpr int MODE = decltype(mode_c)::value;
        if (CACHE > 0) {
#pragma unroll
            for (int c = 0; c < CACHE; ++c) {
                int64_t v = lane + (int64_t)c * TPR;
                if (v < nvec) *reinterpret_cast<uint2 *>(qr + v * 8) = encode8_e4m3<MODE>(cache[c], t);
            }
        } else {
            for (int64_t v = lane; v < nvec; v += TPR)
                *reinterpret_cast<uint2 *>(qr + v * 8) = encode8_e4m3<MODE>(ld16(xr + v * 8), t);
        }
    });
}

// ---------------------------------------------------------------------------
// Per-tensor amax: `parts` blocks per matrix each write the max of their
// slice; the encode kernels fold the partial maxima.  No atomics and no
// zero-initialised scratch, so the result is deterministic.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void amax_partial_kernel(
    const uint16_t *__restrict__ x, int64_t elems, int64_t bstride, int64_t parts,
    uint32_t *__restrict__ partial)
{
    __shared__ uint32_t lds4[4];
    const int64_t b = blockIdx.y;
    const uint16_t *xb = x + b * bstride;
    const int64_t nvec = elems / 8;
    const int64_t per = (nvec + parts - 1) / parts;
    const int64_t v0 = blockIdx.x * per, v1 = min(nvec, v0 + per);
    uint32_t m = 0;
    for (int64_t v = v0 + threadIdx.x; v < v1; v += kThreads) m = max(m, amax8(ld16(xb + v * 8)));
    m = block_max_u32(m, lds4);
    if (threadIdx.x == 0) partial[b * parts + blockIdx.x] = m;
}

__device__ __forceinline__ uint32_t fold_partials(const uint32_t *p, int64_t parts, uint32_t *lds4)
{
    uint32_t m = 0;
    for (int64_t i = threadIdx.x; i < parts; i += kThreads) m = max(m, p[i]);
    return block_max_u32(m, lds4);
}

__global__ __launch_bounds__(kThreads) void quant_tensor_encode_kernel(
    const uint16_t *__restrict__ x, int64_t elems, int64_t bstride, const uint32_t *__restrict__ partial,
    int64_t parts, uint8_t *__restrict__ q, float *__restrict__ scale)
{
    __shared__ uint32_t lds4[4];
    const int64_t b = blockIdx.y;
    const uint32_t m = fold_partials(partial + b * parts, parts, lds4);
    const RowScale t = row_scale(__uint_as_float(m << 16));
    if (blockIdx.x == 0 && threadIdx.x == 0) scale[b] = t.s;
    const uint16_t *xb = x + b * bstride;
    uint8_t *qb = q + b * elems;
    const int64_t nvec = elems / 8;
    with_encode_mode(t, [&](auto mode_c) {
        constexpr int MODE = decltype(mode_c)::value;
        for (int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x; v < nvec; v += (int64_t)gridDim.x * kThreads)
            *reinterpret_cast<uint2 *>(qb + v * 8) = encode8_e4m3<MODE>(ld16(xb + v * 8), t);
    });
}

// ---------------------------------------------------------------------------
// NVFP4 encode of one 16-element group given the tensor scale t: the block
// scale code b = E4M3(fl32(amax_g / fl32(6 t))), e = fl32(dec(b) t), and the
// eight packed code bytes of E2M1(fl32(x / e)) (a zero e gives signed zeros).
// Both NVFP4 quantize kernels use these, so their codes are identical.
// ---------------------------------------------------------------------------

// The E2M1 code of fl32(x / e) from y = fl32(1 / e) (one IEEE division per
// group instead of one per element): q0 = fl32(x y) is within one ulp of
// x / e, the residual x - q0 e is exact (an FMA), and fl32(q0 + r y) is the
// correctly rounded quotient (Markstein's theorem on division by a correctly
// rounded reciprocal, binary arithmetic without underflow or overflow); the
// sign is restored for zeros.  Taken for e in [2^-100, 2^100]; the
// quotients of a group are at most about 12 in magnitude (e is the group
// maximum over 6, rounded to E4M3), so they never overflow, and where x is
// tiny or subnormal an inexact residual can only move a quotient that is
// far below the first E2M1 rounding boundary (0.25).  The E2M1 codes agree
// with those of the division for every bf16 x (zeros and subnormals
// included) over divisors e = fl32(dec(b) t) across the whole range
// (tests/arith/reciprocal_division.c; 1.9e9 cases run once, 4e7 in the CPU
// test suite).  Other e take the division.
__device__ __forceinline__ float div_rn(float x, float e, float y, bool fast_e)
{
#pragma clang fp contract(off)
    if (fast_e) {
        const float q0 = x * y;
        const float r = __builtin_fmaf(-q0, e, x);
        return __builtin_copysignf(__builtin_fmaf(r, y, q0), x);
    }
    return x / e;
}

// Block scale code and element divisor of a group with maximum magnitude
// bits gm (bf16 bits << 16).
struct GroupScale {
    uint32_t b;
    float e, y;
    bool fast;
};

__device__ __forceinline__ GroupScale group_scale(uint32_t gm, float t, float six_t)
{
    GroupScale s;
    s.b = 0;
    if (t > 0.0f) s.b = encode_e4m3(__uint_as_float(gm << 16) / six_t);
    s.e = decode_e4m3(s.b) * t;
    s.fast = s.e >= 0x1p-100f && s.e <= 0x1p100f;
    s.y = s.fast ? 1.0f / s.e : 0.0f;
    return s;
}

// E2M1 codes of eight elements (one 16-byte vector of bf16), packed low
// nibble first: four bytes.  The rounding to E2M1 is v_cvt_scalef32_pk_fp4_f32
// with scale 1 (two quotients per instruction): round to nearest even,
// saturating at +-6, signed zeros kept - the same code as encode_e2m1 for
// every binary32 input that is not a NaN (spg_probe_fp4_rounding checks all
// 2^32 inputs on the device; the quotients here are finite).
__device__ __forceinline__ uint32_t encode_half8(const uint4 &v, const GroupScale &s)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    if (!(s.e > 0.0f)) {   // zero scale: signed zeros
        uint32_t packed = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            packed |= (((w[i] >> 12) & 0x8u) | (((w[i] >> 28) & 0x8u) << 4)) << (8 * i);
        return packed;
    }
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = div_rn(bf16_lo(w[i]), s.e, s.y, s.fast);
        f[2 * i + 1] = div_rn(bf16_hi(w[i]), s.e, s.y, s.fast);
    }
    uint32_t packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, f[0], f[1], 1.0f, 0);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, f[2], f[3], 1.0f, 1);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, f[4], f[5], 1.0f, 2);
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, f[6], f[7], 1.0f, 3);
}

__device__ __forceinline__ void encode_group16(const uint4 &v0, const uint4 &v1, uint32_t gm, float t, float six_t,
                                               uint2 &codes, uint32_t &b)
{
    const GroupScale s = group_scale(gm, t, six_t);
    b = s.b;
    codes = make_uint2(encode_half8(v0, s), encode_half8(v1, s));
}

// Byte offset of block scale (row, group g) in the scale plane.  Row-major:
// row * G + g.  Blocked (the layout the NVFP4 GEMM stages, ninfer PR #160's
// quantizer writing the plane in the tile shape its GEMM reads): the scales of
// 256 rows for one 256-element K stage (16 groups) form one contiguous 4 KiB
// block, row-major inside it, blocks ordered by row tile, then stage; the
// rows of a last, partial row tile are padded with zero bytes.
__device__ __forceinline__ uint64_t scale_offset(uint32_t row, uint32_t g, uint32_t G, int layout)
{
    if (layout == SPG_SCALES_ROW_MAJOR) return (uint64_t)row * G + g;
    return ((uint64_t)(row >> 8) * (G >> 4) + (g >> 4)) * 4096u + (row & 255u) * 16u + (g & 15u);
}

// Two-pass NVFP4, pass 2: fold the partial maxima into t, then encode.  A
// wave takes 64 groups per trip in two windows of 32: lane l loads half
// l % 2 of group l / 2 of each window (16 bytes at 16 l: every load covers
// 1 KiB of whole lines), the lane pair exchanges half-group maxima, the even
// lane forms the scale of its window-0 group and the odd lane that of its
// window-1 group, and they exchange those, so each group's scale is formed
// once.  Each lane stores the four code bytes of its two halves; the even
// lane stores window 0's scale byte, the odd lane window 1's.  Groups past
// the tensor (groups .. groups_pad) get the zero scale bytes of the padding
// rows of a blocked plane.
__global__ __launch_bounds__(kThreads) void quant_block16_encode_kernel(
    const uint16_t *__restrict__ x, int64_t groups, int64_t groups_pad, FastDiv div_g, uint32_t G, int layout,
    const uint32_t *__restrict__ partial, int64_t parts, uint8_t *__restrict__ q, uint8_t *__restrict__ bscale,
    float *__restrict__ tscale)
{
    __shared__ uint32_t lds4[4];
    const uint32_t m = fold_partials(partial, parts, lds4);
    const float t = __uint_as_float(m << 16) / 2688.0f;
    const float six_t = 6.0f * t;
    if (blockIdx.x == 0 && threadIdx.x == 0) *tscale = t;
    const int lane = threadIdx.x & 63, h = lane & 1;
    const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
    const int64_t waves = (int64_t)gridDim.x * (kThreads / 64);
    for (int64_t base = wave * 64; base < groups_pad; base += waves * 64) {
        const int64_t g0 = base + (lane >> 1), g1 = g0 + 32;
        const bool in0 = g0 < groups, in1 = g1 < groups;
        const uint4 v0 = in0 ? ld16(x + g0 * 16 + h * 8) : make_uint4(0u, 0u, 0u, 0u);
        const uint4 v1 = in1 ? ld16(x + g1 * 16 + h * 8) : make_uint4(0u, 0u, 0u, 0u);
        uint32_t m0 = amax8(v0), m1 = amax8(v1);
        m0 = max(m0, (uint32_t)__shfl_xor((int)m0, 1, 64));
        m1 = max(m1, (uint32_t)__shfl_xor((int)m1, 1, 64));
        // this lane's group: window h; the partner's: the other window
        const GroupScale mine = group_scale(h ? m1 : m0, t, six_t);
        GroupScale other;
        other.b = (uint32_t)__shfl_xor((int)mine.b, 1, 64);
        other.e = __shfl_xor(mine.e, 1, 64);
        other.y = __shfl_xor(mine.y, 1, 64);
        other.fast = __shfl_xor((int)mine.fast, 1, 64) != 0;
        const GroupScale &s0 = h ? other : mine, &s1 = h ? mine : other;
        if (in0) *reinterpret_cast<uint32_t *>(q + g0 * 8 + h * 4) = encode_half8(v0, s0);
        if (in1) *reinterpret_cast<uint32_t *>(q + g1 * 8 + h * 4) = encode_half8(v1, s1);
        const int64_t gs = h ? g1 : g0;
        if (gs < groups_pad) {
            const uint32_t row = fdiv_q((uint32_t)gs, div_g), col = (uint32_t)gs - row * G;
            bscale[scale_offset(row, col, G, layout)] = (gs < groups) ? (uint8_t)mine.b : (uint8_t)0;
        }
    }
}

// Single-launch NVFP4 (every block resident: cooperative launch).  Each
// thread loads GPT groups into registers and takes their maxima.  Each block
// stores its maximum in its own slot and counts itself in; the block that
// arrives last is elected, folds the slots into the tensor amax, forms t and
// publishes it with a release flag; the others wait for the flag, then every
// thread encodes its groups straight from registers, so the tensor is read
// from memory once.  Device-scope atomics on one address serialize across
// the XCDs (one counter for 768 blocks measured 135 us for the whole
// quantize), so arrivals are counted in 16 sub-counters on separate cache
// lines; the block completing a sub-counter counts into the top counter.
// The sync area (zeroed by quant_sync_clear_kernel just before) holds the
// 16 sub-counters, the top counter, the flag and t, one 128-byte line each;
// the block maxima follow it.  A wait that runs past spin_limit polls (never
// expected) gives up and publishes a NaN tensor scale instead of hanging.
constexpr int kSubCounters = 16;
constexpr int kLineWords = 32;                              // 128-byte lines
constexpr int kSyncWords = (kSubCounters + 3) * kLineWords; // sub-counters, top, flag, t
constexpr int kFusedThreads = 1024;

__global__ __launch_bounds__(256) void quant_sync_clear_kernel(uint32_t *__restrict__ sync)
{
    for (int i = threadIdx.x; i < kSyncWords; i += 256) sync[i] = 0u;
}

template <int GPT>
__global__ __launch_bounds__(kFusedThreads) void quant_block16_fused_kernel(
    const uint16_t *__restrict__ x, int64_t groups, int64_t groups_pad, FastDiv div_g, uint32_t G, int layout,
    uint8_t *__restrict__ q, uint8_t *__restrict__ bscale, float *__restrict__ tscale, uint32_t *sync,
    int64_t spin_limit)
{
    __shared__ uint32_t lds16[16];
    __shared__ uint32_t t_bits;
    uint32_t *const top = sync + kSubCounters * kLineWords;
    uint32_t *const flag = top + kLineWords;
    uint32_t *const tword = flag + kLineWords;
    uint32_t *const slots = sync + kSyncWords;
    const int64_t nthreads = (int64_t)gridDim.x * kFusedThreads;
    const int64_t tid = (int64_t)blockIdx.x * kFusedThreads + threadIdx.x;
    uint4 v[GPT][2];
    uint32_t gm[GPT];
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < GPT; ++i) {
        const int64_t g = tid + (int64_t)i * nthreads;
        if (g < groups) {
            v[i][0] = ld16(x + g * 16);
            v[i][1] = ld16(x + g * 16 + 8);
        } else {
            v[i][0] = v[i][1] = make_uint4(0, 0, 0, 0);
        }
    }
#pragma unroll
    for (int i = 0; i < GPT; ++i) {
        gm[i] = max(amax8(v[i][0]), amax8(v[i][1]));
        m = max(m, gm[i]);
    }
    // block maximum: wave maxima through LDS
    m = wave_max_u32(m);
    if ((threadIdx.x & 63) == 0) lds16[threadIdx.x >> 6] = m;
    __syncthreads();
    __shared__ uint32_t elected;
    if (threadIdx.x == 0) {
        uint32_t bm = 0;
        for (int w = 0; w < kFusedThreads / 64; ++w) bm = max(bm, lds16[w]);
        __hip_atomic_store(&slots[blockIdx.x], bm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t nb = gridDim.x, j = blockIdx.x % kSubCounters;
        const uint32_t in_j = (nb - j + kSubCounters - 1) / kSubCounters;     // blocks counted by sub-counter j
        const uint32_t nsub = nb < (uint32_t)kSubCounters ? nb : (uint32_t)kSubCounters;
        const uint32_t a = __hip_atomic_fetch_add(&sync[j * kLineWords], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        elected = a == in_j - 1u &&
                  __hip_atomic_fetch_add(top, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) == nsub - 1u;
    }
    __syncthreads();
    if (elected) {
        // every thread of the elected block folds at most one block maximum
        // (gridDim.x <= 1024), then t is formed and published
        uint32_t am = threadIdx.x < gridDim.x
                          ? __hip_atomic_load(&slots[threadIdx.x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                          : 0u;
        am = wave_max_u32(am);
        __syncthreads();
        if ((threadIdx.x & 63) == 0) lds16[threadIdx.x >> 6] = am;
        __syncthreads();
        if (threadIdx.x == 0) {
            for (int w = 0; w < kFusedThreads / 64; ++w) am = max(am, lds16[w]);
            const float t = __uint_as_float(am << 16) / 2688.0f;
            __hip_atomic_store(tword, __float_as_uint(t), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(flag, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (threadIdx.x == 0) {
        // poll with relaxed loads (an acquire load per poll would also
        // invalidate this XCD's caches each time), then acquire once
        int64_t n = 0;
        while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u && n < spin_limit) {
            __builtin_amdgcn_s_sleep(8);
            ++n;
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        t_bits = n < spin_limit ? __hip_atomic_load(tword, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0x7FC00000u;
    }
    __syncthreads();
    const float t = __uint_as_float(t_bits);
    if (blockIdx.x == 0 && threadIdx.x == 0) *tscale = t;
    if (t != t) return;                                      // gave up waiting: NaN published
    const float six_t = 6.0f * t;
#pragma unroll
    for (int i = 0; i < GPT; ++i) {
        const int64_t g = tid + (int64_t)i * nthreads;
        if (g < groups) {
            uint2 codes;
            uint32_t b;
            encode_group16(v[i][0], v[i][1], gm[i], t, six_t, codes, b);
            *reinterpret_cast<uint2 *>(q + g * 8) = codes;
            const uint32_t row = fdiv_q((uint32_t)g, div_g);
            bscale[scale_offset(row, (uint32_t)g - row * G, G, layout)] = (uint8_t)b;
        }
    }
    for (int64_t g = groups + tid; g < groups_pad; g += nthreads) {   // padding rows of a blocked plane
        const uint32_t row = fdiv_q((uint32_t)g, div_g);
        bscale[scale_offset(row, (uint32_t)g - row * G, G, layout)] = 0;
    }
}

int64_t grid_for(int64_t items, int64_t per_block, int64_t cap)
{
    int64_t g = (items + per_block - 1) / per_block;
    return g < 1 ? 1 : (g > cap ? cap : g);
}

}  // namespace

int64_t amax_parts(int64_t elems)
{
    // one partial per 16K elements, at most 1024 per matrix
    int64_t p = (elems + 16383) / 16384;
    return p < 1 ? 1 : (p > 1024 ? 1024 : p);
}

hipError_t launch_quantize_rowwise(const uint16_t *x, int64_t rows, int64_t K, int64_t ldx,
                                   uint8_t *q, int64_t ldq, float *scale, hipStream_t s)
{
    // Short rows: one wave per row, four rows per block.  Longer rows: one
    // 4-wave block per row keeping up to 16 vectors per lane in registers
    // (measured on 4096 x 5120: 13.3 us with 4-wave blocks, 14.7 us with one
    // wave per row), beyond that the encode pass re-reads the row from L2.
    const int64_t nvec = K / 8;
    const dim3 grid64((unsigned)((rows + 3) / 4)), grid256((unsigned)rows);
    if (nvec <= 64 * 1)
        quant_rowwise_kernel<64, 1><<<grid64, kThreads, 0, s>>>(x, rows, K, ldx, q, ldq, scale);
    else if (nvec <= 64 * 2)
        quant_rowwise_kernel<64, 2><<<grid64, kThreads, 0, s>>>(x, rows, K, ldx, q, ldq, scale);
    else if (nvec <= 256 * 1)
        quant_rowwise_kernel<256, 1><<<grid256, kThreads, 0, s>>>(x, rows, K, ldx, q, ldq, scale);
    else if (nvec <= 256 * 2)
        quant_rowwise_kernel<256, 2><<<grid256, kThreads, 0, s>>>(x, rows, K, ldx, q, ldq, scale);
    else if (nvec <= 256 * 4)
        quant_rowwise_kernel<256, 4><<<grid256, kThreads, 0, s>>>(x, rows, K, ldx, q, ldq, scale);
    else if (nvec <= 256 * 8)
        quant_rowwise_kernel<256, 8><<<grid256, kThreads, 0, s>>>(x, rows, K, ldx, q, ldq, scale);
    else if (nvec <= 256 * 16)
        quant_rowwise_kernel<256, 16><<<grid256, kThreads, 0, s>>>(x, rows, K, ldx, q, ldq, scale);
    else
        quant_rowwise_kernel<256, 0><<<grid256, kThreads, 0, s>>>(x, rows, K, ldx, q, ldq, scale);
    return hipGetLastError();
}

hipError_t launch_quantize_tensor(const uint16_t *x, int64_t batch, int64_t rows, int64_t K,
                                  int64_t bstride, uint8_t *q, float *scale, uint32_t *ws,
                                  int64_t parts, hipStream_t s)
{
    const int64_t elems = rows * K;
    amax_partial_kernel<<<dim3((unsigned)parts, (unsigned)batch), kThreads, 0, s>>>(x, elems, bstride, parts, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t g = grid_for(elems / 8, kThreads * 4, 2048);
    quant_tensor_encode_kernel<<<dim3((unsigned)g, (unsigned)batch), kThreads, 0, s>>>(x, elems, bstride, ws,
                                                                                      parts, q, scale);
    return hipGetLastError();
}

namespace {

// Single launch when the whole tensor fits in the registers of one resident
// grid (GPT groups per thread); false (and nothing enqueued but the clear)
// when it does not, or when the cooperative launch is refused.
static_assert(kBlock16SyncWords >= kSyncWords + kMaxFusedBlocks, "sync area too small");

// Blocks of the single-launch kernel for `groups` groups, or 0 when they
// cannot all be resident at once on the current device.
template <int GPT>
int64_t fused_blocks(int64_t groups)
{
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, quant_block16_fused_kernel<GPT>, kFusedThreads, 0) !=
            hipSuccess || per_cu <= 0)
        return 0;
    const int64_t need = (groups + (int64_t)kFusedThreads * GPT - 1) / ((int64_t)kFusedThreads * GPT);
    return need <= (int64_t)cus * per_cu && need <= kMaxFusedBlocks ? need : 0;
}

template <int GPT>
bool try_fused_block16(const uint16_t *x, int64_t groups, int64_t groups_pad, FastDiv div_g, uint32_t G, int layout,
                       uint8_t *q, uint8_t *bscale, float *tscale, uint32_t *sync, hipStream_t s)
{
    const int64_t need = fused_blocks<GPT>(groups);
    if (need == 0) return false;
    quant_sync_clear_kernel<<<1, 256, 0, s>>>(sync);
    if (hipGetLastError() != hipSuccess) return false;
    int64_t spin_limit = INT64_C(1) << 22;
    void *args[] = {(void *)&x, (void *)&groups, (void *)&groups_pad, (void *)&div_g, (void *)&G, (void *)&layout,
                    (void *)&q, (void *)&bscale, (void *)&tscale, (void *)&sync, (void *)&spin_limit};
    if (hipLaunchCooperativeKernel((const void *)quant_block16_fused_kernel<GPT>, dim3((unsigned)need),
                                   dim3(kFusedThreads), args, 0, s) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return true;
}

}  // namespace

bool quantize_block16_single_launch(int64_t rows, int64_t K)
{
    const int64_t groups = rows * K / 16;
    return fused_blocks<8>(groups) > 0;
}

hipError_t launch_quantize_block16(const uint16_t *x, int64_t rows, int64_t K, uint8_t *q,
                                   uint8_t *bscale, float *tscale, int layout, bool single_launch, uint32_t *ws,
                                   int64_t parts, hipStream_t s)
{
    const int64_t elems = rows * K;
    const int64_t groups = elems / 16;
    const uint32_t G = (uint32_t)(K / 16);
    const int64_t rows_pad = layout == SPG_SCALES_BLOCKED ? (rows + 255) / 256 * 256 : rows;
    const int64_t groups_pad = rows_pad * G;
    const FastDiv div_g = make_fastdiv(G);
    uint32_t *sync = ws, *partial = ws + kBlock16SyncWords;
    if (single_launch && try_fused_block16<8>(x, groups, groups_pad, div_g, G, layout, q, bscale, tscale, sync, s))
        return hipGetLastError();
    // two passes: partial maxima, then fold and encode (reads the tensor again)
    amax_partial_kernel<<<dim3((unsigned)parts, 1), kThreads, 0, s>>>(x, elems, elems, parts, partial);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t g = grid_for(groups_pad, kThreads * 2, 4096);
    quant_block16_encode_kernel<<<dim3((unsigned)g), kThreads, 0, s>>>(x, groups, groups_pad, div_g, G, layout, partial,
                                                                      parts, q, bscale, tscale);
    return hipGetLastError();
}

}  // namespace spg
