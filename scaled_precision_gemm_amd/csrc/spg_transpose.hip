// Byte transpose of FP8 codes for K-major operands (spg_layout): a stored
// [R, C] code matrix (row stride ld, batch stride bstride) becomes [C, R]
// with row stride R, which the NT GEMM kernels then read K-contiguous.
//
// One workgroup per 64 x 64 block of one batch entry: 256 threads each load
// 16 bytes of a source row (4 per row, coalesced 64-byte row segments), the
// block goes through LDS, and each thread gathers 16 bytes of one source
// column (16 consecutive source rows) and stores them as one 16-byte piece
// of a destination row.  HBM-bound: each byte is read and written once.
#include "spg_common.h"

namespace spg {

namespace {

constexpr int kTB = 64;            // block edge (bytes)
constexpr int kTPad = kTB + 4;     // LDS row pitch: a column gather walks rows 68 bytes apart

// One-dimensional grid of nbc * nbr * batch blocks (block columns fastest).
__global__ __launch_bounds__(256) void transpose_u8_kernel(const uint8_t *src, int64_t R, int64_t C, int64_t ld,
                                                          int64_t bstride, uint8_t *dst, uint32_t nbc, uint32_t nbr)
{
    __shared__ uint8_t tile[kTB * kTPad];
    const int t = threadIdx.x;
    const uint32_t bid = blockIdx.x, per = nbc * nbr;
    const int64_t b = bid / per;
    const uint32_t rem = bid - (uint32_t)b * per;
    const int64_t r0 = (int64_t)(rem / nbc) * kTB, c0 = (int64_t)(rem % nbc) * kTB;
    const uint8_t *s = src + b * bstride;
    uint8_t *d = dst + b * R * C;

    // load: source row r0 + t / 4, bytes c0 + 16 (t % 4) .. + 15
    {
        const int r = t >> 2, cc = (t & 3) * 16;
        const int64_t row = r0 + r, col = c0 + cc;
        uint8_t v[16];
        if (row < R && col + 16 <= C) {
            const uint4 q = *reinterpret_cast<const uint4 *>(s + row * ld + col);   // 16-byte aligned
            const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] = (uint8_t)(w[i >> 2] >> (8 * (i & 3)));
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] = (row < R && col + i < C) ? s[row * ld + col + i] : 0;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) tile[r * kTPad + cc + i] = v[i];
    }
    __syncthreads();

    // store: destination row c0 + t / 4 (source column), bytes r0 + 16 (t % 4) .. + 15
    {
        const int oc = t >> 2, rc = (t & 3) * 16;
        const int64_t orow = c0 + oc, ocol = r0 + rc;
        if (orow >= C) return;
        uint8_t v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = tile[(rc + i) * kTPad + oc];
        uint8_t *out = d + orow * R + ocol;
        if (ocol + 16 <= R) {
            uint32_t w[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                w[j] = (uint32_t)v[4 * j] | (uint32_t)v[4 * j + 1] << 8 | (uint32_t)v[4 * j + 2] << 16 |
                       (uint32_t)v[4 * j + 3] << 24;
            *reinterpret_cast<uint4 *>(out) = make_uint4(w[0], w[1], w[2], w[3]);   // R % 16 == 0
        } else {
            for (int i = 0; i < 16 && ocol + i < R; ++i) out[i] = v[i];
        }
    }
}

}  // namespace

hipError_t launch_transpose_u8(const uint8_t *src, int64_t R, int64_t C, int64_t ld, int64_t bstride,
                               int64_t batch, uint8_t *dst, hipStream_t s)
{
    if (R == 0 || C == 0 || batch == 0) return hipSuccess;
    const int64_t nbc = (C + kTB - 1) / kTB, nbr = (R + kTB - 1) / kTB;
    if (nbc * nbr * batch >= (INT64_C(1) << 31)) return hipErrorInvalidValue;   // checked by the caller
    transpose_u8_kernel<<<dim3((unsigned)(nbc * nbr * batch)), 256, 0, s>>>(src, R, C, ld, bstride, dst,
                                                                            (uint32_t)nbc, (uint32_t)nbr);
    return hipGetLastError();
}

}  // namespace spg
