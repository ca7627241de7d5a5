// Measurement probes: the machine's own ceilings, quoted next to the GEMM and
// quantizer figures.  They are not steps of the method.
//
//  * MFMA-only: every wave runs back-to-back MFMAs on register operands
//    (four independent accumulator chains, so no MFMA waits for the result
//    of the one before), as ninfer PR #160 measured the fed ceiling of its
//    own MMA in its summary - here for the instructions the GEMM kernels
//    use: E4M3 x E4M3 32x32x64 and f16 32x32x16.  Operands are fixed pseudo-random bit patterns with no
//    NaN or infinity, because the power controller reacts to operand
//    activity (constant operands run at a higher clock than random ones).
//    Wave 0 of workgroup 0 reads the shader-clock counter (s_memtime) and the
//    fixed 100 MHz counter (s_memrealtime) around its loop, which gives the
//    shader clock the MFMAs ran at.
//  * HBM read: a grid-stride stream of 16-byte loads over a buffer larger
//    than the last-level cache, folded with XOR into one word per thread (the
//    folded words are checkable against the buffer).
//  * FP4 rounding: the NVFP4 quantizers round quotients to E2M1 with
//    v_cvt_scalef32_pk_fp4_f32 (scale 1); this probe compares that
//    instruction with the library's E2M1 encoder for every binary32 input
//    that is not a NaN (2^32 - 2^24 values) and counts the differences.
#include "spg_common.h"

namespace spg {

namespace {

constexpr int kProbeThreads = 256;

__device__ __forceinline__ uint32_t mix32(uint32_t x)
{
    // a 32-bit integer hash (xorshift-multiply), only to spread bits
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return x;
}

template <int KIND>
__global__ __launch_bounds__(kProbeThreads) void probe_mfma_kernel(int64_t iters, float *sink, uint64_t *clocks)
{
    const uint32_t tid = blockIdx.x * kProbeThreads + threadIdx.x;
    // E4M3: clearing bit 3 of every byte keeps exponent fields even, so no
    // byte is 0x7F / 0xFF (NaN).  f16: clearing bit 14 of every half keeps
    // exponents below 16 (|v| < 2), no infinity or NaN.
    const uint32_t mask = KIND == 0 ? 0xF7F7F7F7u : 0xBFFFBFFFu;
    v8i a[4], b[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a[c][e] = (int)(mix32(tid * 64u + (uint32_t)(c * 8 + e)) & mask);
            b[c][e] = (int)(mix32(tid * 64u + 32u + (uint32_t)(c * 8 + e)) & mask);
        }
    v16f acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[c][e] = 0.0f;

    const bool timer = blockIdx.x == 0 && threadIdx.x < 64;
    uint64_t t0 = 0, r0 = 0;
    if (timer) {
        t0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
    }
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (KIND == 0) {
                acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[c], b[c], acc[c], 0, 0, 0, 0, 0, 0);
            } else {
                typedef _Float16 h8 __attribute__((ext_vector_type(8)));
                const v4i a4 = {a[c][0], a[c][1], a[c][2], a[c][3]};
                const v4i b4 = {b[c][0], b[c][1], b[c][2], b[c][3]};
                acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8, a4), __builtin_bit_cast(h8, b4),
                                                                acc[c], 0, 0, 0);
            }
        }
    }
    if (timer) {
        const uint64_t t1 = __builtin_amdgcn_s_memtime();
        const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
        if (threadIdx.x == 0) {
            clocks[0] = t0;
            clocks[1] = t1;
            clocks[2] = r0;
            clocks[3] = r1;
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[c][e];
    sink[tid] = s;
}

__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const v4i *__restrict__ src, int64_t n16,
                                                                   uint32_t *__restrict__ sink)
{
    const int64_t tid = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
    uint32_t x = 0;
    int64_t i = tid;
    // four loads in flight per thread
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const v4i v0 = __builtin_nontemporal_load(src + i);
        const v4i v1 = __builtin_nontemporal_load(src + i + stride);
        const v4i v2 = __builtin_nontemporal_load(src + i + 2 * stride);
        const v4i v3 = __builtin_nontemporal_load(src + i + 3 * stride);
        const v4i v = v0 ^ v1 ^ v2 ^ v3;
        x ^= (uint32_t)(v[0] ^ v[1] ^ v[2] ^ v[3]);
    }
    for (; i < n16; i += stride) {
        const v4i v = src[i];
        x ^= (uint32_t)(v[0] ^ v[1] ^ v[2] ^ v[3]);
    }
    sink[tid] = x;
}

__global__ __launch_bounds__(64) void probe_clear_kernel(uint32_t *out, int n)
{
    if ((int)threadIdx.x < n) out[threadIdx.x] = 0u;
}

// Thread t checks the 256 inputs 256 t .. 256 t + 255 (two per conversion);
// out[0] counts differences, out[1] the recorded ones, and the first 16 are
// kept as (input bits, instruction code | encoder code << 8).
__global__ __launch_bounds__(kProbeThreads) void probe_fp4_kernel(uint32_t *out)
{
    const uint32_t u0 = (uint32_t)(((uint64_t)blockIdx.x * kProbeThreads + threadIdx.x) * 256u);
    uint32_t bad = 0;
    for (uint32_t i = 0; i < 256; i += 2) {
        const uint32_t ua = u0 + i, ub = ua + 1;
        const uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, __uint_as_float(ua), __uint_as_float(ub),
                                                                    1.0f, 0);
        const uint32_t us[2] = {ua, ub};
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if ((us[j] & 0x7FFFFFFFu) > 0x7F800000u) continue;   // NaN
            const uint32_t got = (r >> (4 * j)) & 0xFu, want = encode_e2m1(__uint_as_float(us[j]));
            if (got != want) {
                ++bad;
                const uint32_t k = atomicAdd(&out[1], 1u);
                if (k < 16) {
                    out[2 + 2 * k] = us[j];
                    out[3 + 2 * k] = got | (want << 8);
                }
            }
        }
    }
    if (bad) atomicAdd(&out[0], bad);
}

}  // namespace

}  // namespace spg

using namespace spg;

SPG_EXPORT int spg_probe_fp4_rounding(uint32_t *result, void *stream)
{
    if (!result || ((uintptr_t)result & 3)) return SPG_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    probe_clear_kernel<<<1, 64, 0, s>>>(result, 34);
    if (hipGetLastError() != hipSuccess) return SPG_EHIP;
    // 65536 workgroups x 256 threads x 256 inputs = every 32-bit pattern
    probe_fp4_kernel<<<dim3(65536), kProbeThreads, 0, s>>>(result);
    return hipGetLastError() == hipSuccess ? SPG_OK : SPG_EHIP;
}

SPG_EXPORT int spg_probe_mfma(int kind, int64_t iters, int32_t workgroups, float *sink, uint64_t *clocks,
                              void *stream)
{
    if ((kind != 0 && kind != 1) || iters < 1 || workgroups < 1 || !sink || !clocks) return SPG_EINVAL;
    if (((uintptr_t)sink & 3) || ((uintptr_t)clocks & 7)) return SPG_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    if (kind == 0)
        probe_mfma_kernel<0><<<dim3((unsigned)workgroups), kProbeThreads, 0, s>>>(iters, sink, clocks);
    else
        probe_mfma_kernel<1><<<dim3((unsigned)workgroups), kProbeThreads, 0, s>>>(iters, sink, clocks);
    return hipGetLastError() == hipSuccess ? SPG_OK : SPG_EHIP;
}

SPG_EXPORT int spg_probe_read(const void *src, int64_t bytes, int32_t workgroups, uint32_t *sink, void *stream)
{
    if (!src || !sink || bytes < 16 || (bytes & 15) || workgroups < 1) return SPG_EINVAL;
    if (((uintptr_t)src & 15) || ((uintptr_t)sink & 3)) return SPG_EINVAL;
    probe_read_kernel<<<dim3((unsigned)workgroups), kProbeThreads, 0, (hipStream_t)stream>>>(
        (const v4i *)src, bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? SPG_OK : SPG_EHIP;
}
