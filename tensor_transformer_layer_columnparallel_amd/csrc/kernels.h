// Internal launch interface between the C entry points and the kernels.
#pragma once

#include "common.h"

namespace tpmlp {

// Operand layouts of C = op(A) op(B), named by whether each operand is used
// as stored ("N": A [M][K], B [K][N]) or transposed ("T").
//   NN: A [M][K] K-contiguous, B [K][N] N-contiguous   (forward products)
//   NT: A [M][K] K-contiguous, B [N][K] K-contiguous   (x W^T products)
//   TN: A [K][M] M-contiguous, B [K][N] N-contiguous   (x^T dy products)
enum class Layout { NN = 0, NT = 1, TN = 2 };

// General kernel: any layout, fp32 or bf16, any M (ragged tiles masked).
hipError_t gemm_simple(const GemmArgs& p, Elt elt, Layout layout, Epi epi, Elt out,
                       hipStream_t stream);

// 256 x 192-tile bf16 kernel: LDS-DMA into rings of 64-deep units (a
// K-contiguous A) and 32-deep slabs (the other operands), transposed LDS
// reads for M/N-contiguous operands, XCD-aware tile order.
bool gemm_ring_supported(const GemmArgs& p, Layout layout);
hipError_t gemm_ring(const GemmArgs& p, Layout layout, Epi epi, Elt out, hipStream_t stream);
// Rows of C per tile of the tile kernel (the row blocks of GemmArgs::colsum).
constexpr int64_t kGemmRingTileRows = 256;

// out[c][r] = in[r][c] for 16-bit elements, in [rows][cols] (cols % 8 == 0).
// With col_part non-null the same launch also does column_finish(col_part,
// col_out, col_parts, col_count) (below): the backward runs the bias
// gradient's last pass beside the transpose that follows the dY product.
hipError_t transpose16(const void* in, void* out, int64_t rows, int64_t cols, hipStream_t stream,
                       const float* col_part = nullptr, float* col_out = nullptr,
                       int64_t col_parts = 0, int64_t col_count = 0);

// out[e] = sum_{r=0}^{t-1} parts[r][e] (fp32, rank order), parts[r] at
// element offset r * stride; count % 8 == 0 and stride % 8 == 0.
hipError_t shard_sum(const void* parts, void* out, int64_t count, int64_t stride, int t, Elt in,
                     Elt out_elt, hipStream_t stream);

// y[m][:] = (x[m][:] - mean) / sqrt(var + eps) * gamma + beta over each row
// (biased variance, fp32 statistics, fixed reduction order); gamma and beta
// (element type of y) may be null; cols % 8 == 0.
hipError_t layernorm(const void* x, const void* gamma, const void* beta, void* y, int64_t rows,
                     int64_t cols, float eps, Elt in, Elt out, hipStream_t stream);

// The layer norm above of rows that are sums of t partials: row m is
// sum_{r=0}^{t-1} parts[r * stride + m * cols + c] (fp32, rank order), the
// values shard_sum writes with an fp32 output, normalised without being
// stored.  rows = the rank's token rows; parts points at its first row.
hipError_t sum_layernorm(const void* parts, int64_t stride, int t, const void* gamma,
                         const void* beta, void* y, int64_t rows, int64_t cols, float eps, Elt in,
                         Elt out, hipStream_t stream);

// out[m][r*cols + c] = parts[r][m][c]; cols % 8 == 0.
hipError_t shard_concat(const void* parts, void* out, int64_t rows, int64_t cols, int t,
                        Elt elt, hipStream_t stream);

// out[j] = sum_m in[m][j] in fp32, fixed summation order: the bias gradient.
// With scratch of at least ceil(rows / 64) * cols floats it sums row blocks
// of 64 first (more parallel), otherwise one pass per column block.
hipError_t column_sum(const void* in, float* out, int64_t rows, int64_t cols, Elt elt,
                      void* scratch, int64_t scratch_bytes, hipStream_t stream);

// out[j] = sum_r part[r][j] for r = 0 .. nparts - 1 in order: the last step of
// a column sum whose row-block partials another kernel wrote.
hipError_t column_finish(const float* part, float* out, int64_t nparts, int64_t cols,
                         hipStream_t stream);

// One column of column_finish (every kernel that runs it adds in this order).
__device__ __forceinline__ void column_finish_one(const float* __restrict__ part,
                                                  float* __restrict__ out, int64_t nparts,
                                                  int64_t cols, int64_t c)
{
    float acc = 0.f;
    int64_t rb = 0;
    for (; rb + 8 <= nparts; rb += 8) {   // eight loads in flight, adds in order
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = part[(rb + u) * cols + c];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += v[u];
    }
    for (; rb < nparts; ++rb) acc += part[rb * cols + c];
    out[c] = acc;
}

}  // namespace tpmlp
