// out[c][r] = in[r][c] for a 16-bit matrix of rows x cols: 64 x 64 tiles
// staged through LDS, so that both the reads and the writes move whole
// 128-byte row segments.  Used to turn the x^T dy products of the backward
// into products whose first operand is K-contiguous.
#include "common.h"
#include "kernels.h"

namespace tpmlp {
namespace {

constexpr int kTile = 64;
constexpr int kThreads = 256;
constexpr int kPad = 2;   // row stride 66 elements: column reads spread over banks

struct Vec16 {
    uint32_t w[8];   // 16 consecutive 16-bit elements
};

__global__ __launch_bounds__(kThreads) void transpose16_kernel(const uint16_t* __restrict__ in,
                                                               uint16_t* __restrict__ out,
                                                               int64_t rows, int64_t cols,
                                                               int64_t tiles_c)
{
    __shared__ __attribute__((aligned(16))) uint16_t t[kTile][kTile + kPad];
    const int64_t tile = blockIdx.x;
    const int64_t r0 = (tile / tiles_c) * kTile, c0 = (tile % tiles_c) * kTile;
    const int tid = threadIdx.x;

    // Read: thread -> row tid / 4, 16 columns from 16 (tid % 4).
    {
        const int r = tid >> 2, c = (tid & 3) * 16;
        const int64_t gr = r0 + r, gc = c0 + c;
        Vec16 v;
        if (gr < rows && gc + 16 <= cols) {
            const uint4* p = reinterpret_cast<const uint4*>(in + gr * cols + gc);
            const uint4 a = p[0], b = p[1];
            v = Vec16{{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w}};
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t lo = (gr < rows && gc + 2 * j < cols) ? in[gr * cols + gc + 2 * j] : 0u;
                const uint32_t hi =
                    (gr < rows && gc + 2 * j + 1 < cols) ? in[gr * cols + gc + 2 * j + 1] : 0u;
                v.w[j] = lo | (hi << 16);
            }
        }
        uint32_t* row = reinterpret_cast<uint32_t*>(&t[r][c]);
#pragma unroll
        for (int j = 0; j < 8; ++j) row[j] = v.w[j];
    }
    __syncthreads();

    // Write: thread -> output row (input column) tid / 4, 16 input rows from
    // 16 (tid % 4).
    {
        const int c = tid >> 2, r = (tid & 3) * 16;
        const int64_t gc = c0 + c, gr = r0 + r;
        if (gc >= cols) return;
        Vec16 v;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            v.w[j] = (uint32_t)t[r + 2 * j][c] | ((uint32_t)t[r + 2 * j + 1][c] << 16);
        uint16_t* q = out + gc * rows + gr;
        if (gr + 16 <= rows && rows % 8 == 0) {
            uint4* p = reinterpret_cast<uint4*>(q);
            p[0] = uint4{v.w[0], v.w[1], v.w[2], v.w[3]};
            p[1] = uint4{v.w[4], v.w[5], v.w[6], v.w[7]};
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j)
                if (gr + j < rows) q[j] = (uint16_t)(v.w[j >> 1] >> (16 * (j & 1)));
        }
    }
}

}  // namespace

hipError_t transpose16(const void* in, void* out, int64_t rows, int64_t cols, hipStream_t stream)
{
    if (rows == 0 || cols == 0) return hipSuccess;
    const int64_t tiles_r = (rows + kTile - 1) / kTile, tiles_c = (cols + kTile - 1) / kTile;
    if (tiles_r * tiles_c > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(transpose16_kernel, dim3((unsigned)(tiles_r * tiles_c)), dim3(kThreads), 0,
                       stream, static_cast<const uint16_t*>(in), static_cast<uint16_t*>(out),
                       rows, cols, tiles_c);
    return hipGetLastError();
}

}  // namespace tpmlp
