// out[c][r] = in[r][c] for a 16-bit matrix of rows x cols.  Each lane moves an
// 8 x 8 block through its registers (eight 16-byte row loads, 32 byte
// permutes, eight 16-byte column stores); the eight lanes of a block row
// cover 128 contiguous bytes on both sides, so reads and writes move whole
// 128-byte segments.  Used to turn the x^T dy products of the backward into
// products whose first operand is K-contiguous.
#include "common.h"
#include "kernels.h"

namespace tpmlp {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;            // one wave: 64 x 64 elements, 8 x 8 blocks of 8 x 8
constexpr int kWavesPerBlock = kThreads / 64;

__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b)
{
    return (a & 0xffffu) | (b << 16);   // low halves of a and b
}
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b)
{
    return (a >> 16) | (b & 0xffff0000u);   // high halves of a and b
}

// Blocks from tblocks on do the column-finish job (one column per thread).
__global__ __launch_bounds__(kThreads) void transpose16_kernel(const uint16_t* __restrict__ in,
                                                               uint16_t* __restrict__ out,
                                                               int64_t rows, int64_t cols,
                                                               int64_t tiles_c, int64_t ntiles,
                                                               int64_t tblocks,
                                                               const float* __restrict__ col_part,
                                                               float* __restrict__ col_out,
                                                               int64_t col_parts, int64_t col_count)
{
    if ((int64_t)blockIdx.x >= tblocks) {
        const int64_t c = ((int64_t)blockIdx.x - tblocks) * kThreads + threadIdx.x;
        if (c < col_count) column_finish_one(col_part, col_out, col_parts, col_count, c);
        return;
    }
    const int lane = threadIdx.x & 63;
    const int64_t tile = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    if (tile >= ntiles) return;
    // Lane -> 8 x 8 block: input rows 8 (lane % 8) .., input columns 8 (lane / 8) ..
    const int64_t r = (tile / tiles_c) * kTile + 8 * (lane & 7);
    const int64_t c = (tile % tiles_c) * kTile + 8 * (lane >> 3);
    if (c >= cols) return;   // cols % 8 == 0: a block is all in or all out

    uint32_t w[8][4];   // w[i][k]: input row r + i, columns c + 2k, c + 2k + 1
    if (r + 8 <= rows) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint4 v = *reinterpret_cast<const uint4*>(in + (r + i) * cols + c);
            w[i][0] = v.x; w[i][1] = v.y; w[i][2] = v.z; w[i][3] = v.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint4 v = {0u, 0u, 0u, 0u};
            if (r + i < rows) v = *reinterpret_cast<const uint4*>(in + (r + i) * cols + c);
            w[i][0] = v.x; w[i][1] = v.y; w[i][2] = v.z; w[i][3] = v.w;
        }
    }
    // Output row c + j holds input rows r .. r + 7 of column c + j.
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t o[4];
#pragma unroll
        for (int m = 0; m < 4; ++m)
            o[m] = (j & 1) ? hi_pair(w[2 * m][j >> 1], w[2 * m + 1][j >> 1])
                           : lo_pair(w[2 * m][j >> 1], w[2 * m + 1][j >> 1]);
        uint16_t* q = out + (c + j) * rows + r;
        if (r + 8 <= rows && rows % 8 == 0) {
            *reinterpret_cast<uint4*>(q) = uint4{o[0], o[1], o[2], o[3]};
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (r + e < rows) q[e] = (uint16_t)(o[e >> 1] >> (16 * (e & 1)));
        }
    }
}

}  // namespace

hipError_t transpose16(const void* in, void* out, int64_t rows, int64_t cols, hipStream_t stream,
                       const float* col_part, float* col_out, int64_t col_parts,
                       int64_t col_count)
{
    if (!col_part) col_count = 0;
    const int64_t tiles_r = (rows + kTile - 1) / kTile, tiles_c = (cols + kTile - 1) / kTile;
    const int64_t ntiles = rows > 0 && cols > 0 ? tiles_r * tiles_c : 0;
    const int64_t tblocks = (ntiles + kWavesPerBlock - 1) / kWavesPerBlock;
    const int64_t blocks = tblocks + (col_count + kThreads - 1) / kThreads;
    if (blocks == 0) return hipSuccess;
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(transpose16_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(in), static_cast<uint16_t*>(out), rows, cols,
                       tiles_c, ntiles, tblocks, col_part, col_out, col_parts, col_count);
    return hipGetLastError();
}

}  // namespace tpmlp
