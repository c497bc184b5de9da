/*
 * fp64 CPU oracle for one tensor-parallel rank's share of a transformer MLP.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * statement of what the GPU path computes.  Only the test suite, the smoke
 * check and the CPU-baseline leg of the benchmark may load it.  It shares no
 * code, header, table or constant with the HIP library and includes nothing
 * from it.
 *
 * Every quantity is double precision.  Inputs arrive already widened from
 * their storage type (bf16 or fp32 values are exactly representable in fp64),
 * and no intermediate result is rounded.  All matrices are row-major; a
 * weight shard is stored [in_features, out_features/t] and used as x @ W, the
 * convention of the PyTorch example on the page "张量并行实战：从理论到PyTorch
 * 代码的完整落地指南" (section "PyTorch 实现示例：自定义张量并行 Linear 层").
 *
 * Sources for each definition (page title, then section):
 *   [P1] "PaddlePaddle张量并行：从原理到工业落地的深度解析" - introduction:
 *        column split Y_i = X W_i, results joined by AllGather; the input
 *        gradient is aggregated over devices (ReduceScatter / AllReduce).
 *   [P2] "张量并行是什么：2026 大模型训练核心原理与实战详解" - section
 *        "核心工作机制：切分矩阵，协同计算": column-parallel layer followed by a
 *        row-parallel layer whose shard input is the column layer's output.
 *   [P3] "张量并行实战" - section "PyTorch 实现示例": local x @ W + b, then
 *        all_gather and concatenation along the last dimension in rank order.
 *   [P4] "Tensor Parallelism原理与实践：大模型训练的关键技术" - §2.1 (block
 *        matrix product and distributivity), §3.1 (column backward
 *        dL/dW_i = X^T dL/dY_i; row backward dL/dX_i = dL/dY W_i^T).
 *
 * The activation is the tanh approximation of GeLU (Hendrycks & Gimpel,
 * "Gaussian Error Linear Units", 2016).  The pages name only "an activation
 * function"; the tanh form is the reading used throughout this project.
 *
 * Loops are parallelised over independent output rows with OpenMP; within
 * one output element the sum runs over the contraction index in ascending
 * order.  No blocking, reordering or fusion beyond that.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_API __attribute__((visibility("default")))

/* sqrt(2/pi) and the cubic coefficient of the tanh form of GeLU
 * (Hendrycks & Gimpel 2016, section 2). */
static double gelu_scale(void) { return sqrt(2.0 / M_PI); }
static const double GELU_CUBIC = 0.044715;

/* g(y) = 0.5 y (1 + tanh(sqrt(2/pi) (y + 0.044715 y^3))) */
static double gelu_tanh(double y)
{
    double u = gelu_scale() * (y + GELU_CUBIC * y * y * y);
    return 0.5 * y * (1.0 + tanh(u));
}

/* g'(y), by the product and chain rules applied to g above:
 *   g'(y) = 0.5 (1 + tau) + 0.5 y (1 - tau^2) sqrt(2/pi) (1 + 3 * 0.044715 y^2),
 *   tau   = tanh(sqrt(2/pi) (y + 0.044715 y^3)). */
static double gelu_tanh_grad(double y)
{
    double u = gelu_scale() * (y + GELU_CUBIC * y * y * y);
    double tau = tanh(u);
    double du = gelu_scale() * (1.0 + 3.0 * GELU_CUBIC * y * y);
    return 0.5 * (1.0 + tau) + 0.5 * y * (1.0 - tau * tau) * du;
}

ORACLE_API void oracle_gelu_tanh(const double* y, double* out, int64_t count)
{
    for (int64_t i = 0; i < count; ++i) out[i] = gelu_tanh(y[i]);
}

ORACLE_API void oracle_gelu_tanh_grad(const double* y, double* out, int64_t count)
{
    for (int64_t i = 0; i < count; ++i) out[i] = gelu_tanh_grad(y[i]);
}

/* C[m][j] = sum_k A[m][k] * B[k][j]            A [M,K], B [K,N], C [M,N] */
ORACLE_API void oracle_matmul(const double* A, const double* B, double* C,
                              int64_t M, int64_t K, int64_t N)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        double* c = C + m * N;
        for (int64_t j = 0; j < N; ++j) c[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = A[m * K + k];
            const double* b = B + k * N;
            for (int64_t j = 0; j < N; ++j) c[j] += a * b[j];
        }
    }
}

/* Column-parallel linear on one shard [P3 "PyTorch 实现示例", P4 §2.1]:
 *   Y_i[m][j] = sum_k X[m][k] W_i[k][j] + b_i[j]      (b_i may be NULL = 0)
 * Optionally followed by the activation: H_i = g(Y_i). */
ORACLE_API void oracle_column_linear(const double* X, const double* W_i, const double* b_i,
                                     double* Y_i, int64_t tokens, int64_t in_features,
                                     int64_t out_local, int apply_gelu)
{
    oracle_matmul(X, W_i, Y_i, tokens, in_features, out_local);
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < tokens; ++m) {
        double* y = Y_i + m * out_local;
        for (int64_t j = 0; j < out_local; ++j) {
            double v = y[j] + (b_i ? b_i[j] : 0.0);
            y[j] = apply_gelu ? gelu_tanh(v) : v;
        }
    }
}

/* Row-parallel partial product [P2 "核心工作机制", P4 §3.1 row parallel]:
 *   Z_i[m][c] = sum_j X_i[m][j] W_i[j][c]        (no bias on the partial) */
ORACLE_API void oracle_row_linear(const double* X_i, const double* W_i, double* Z_i,
                                  int64_t tokens, int64_t in_local, int64_t out_features)
{
    oracle_matmul(X_i, W_i, Z_i, tokens, in_local, out_features);
}

/* Forward of one MLP shard: the column layer's output shard is the row
 * layer's input shard, so no exchange sits between them [P2 "核心工作机制"].
 *   Y_i = X W1_i + b1_i,  H_i = g(Y_i),  Z_i = H_i W2_i
 * X [T,h], W1_i [h,n], b1_i [n] (NULL = 0), W2_i [n,h];
 * Y_i, H_i [T,n]; Z_i [T,h]. */
ORACLE_API void oracle_mlp_shard_fwd(const double* X, const double* W1_i, const double* b1_i,
                                     const double* W2_i, double* Y_i, double* H_i, double* Z_i,
                                     int64_t T, int64_t h, int64_t n)
{
    oracle_column_linear(X, W1_i, b1_i, Y_i, T, h, n, 0);
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < T; ++m)
        for (int64_t j = 0; j < n; ++j) H_i[m * n + j] = gelu_tanh(Y_i[m * n + j]);
    oracle_row_linear(H_i, W2_i, Z_i, T, n, h);
}

/* Backward of one MLP shard, given the full output gradient dZ (replicated on
 * every rank) and the shard's forward values Y_i, H_i:
 *   dH_i  = dZ W2_i^T                     row layer, dL/dX_i = dL/dY W_i^T [P4 §3.1]
 *   dY_i  = dH_i (elementwise) g'(Y_i)    chain rule through the activation
 *   dW2_i = H_i^T dZ                      dL/dW_i = X^T dL/dY_i [P4 §3.1]
 *   dW1_i = X^T dY_i                      same rule, column layer [P4 §3.1]
 *   dX_i  = dY_i W1_i^T                   this rank's share of the input
 *                                         gradient, summed over ranks [P1]
 *   db1_i = sum over tokens of dY_i       bias gradient (chain rule through
 *                                         Y_i = X W1_i + b1_i); db1_i may be NULL
 * Shapes: dZ [T,h]; dY_i [T,n]; dW2_i [n,h]; dW1_i [h,n]; dX_i [T,h]; db1_i [n]. */
ORACLE_API void oracle_mlp_shard_bwd(const double* X, const double* W1_i, const double* W2_i,
                                     const double* Y_i, const double* H_i, const double* dZ,
                                     double* dY_i, double* dW2_i, double* dW1_i, double* dX_i,
                                     double* db1_i, int64_t T, int64_t h, int64_t n)
{
    /* dY_i[m][j] = (sum_c dZ[m][c] W2_i[j][c]) * g'(Y_i[m][j]) */
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < T; ++m) {
        for (int64_t j = 0; j < n; ++j) {
            double s = 0.0;
            for (int64_t c = 0; c < h; ++c) s += dZ[m * h + c] * W2_i[j * h + c];
            dY_i[m * n + j] = s * gelu_tanh_grad(Y_i[m * n + j]);
        }
    }
    /* dW2_i[j][c] = sum_m H_i[m][j] dZ[m][c] */
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        double* w = dW2_i + j * h;
        for (int64_t c = 0; c < h; ++c) w[c] = 0.0;
        for (int64_t m = 0; m < T; ++m) {
            const double a = H_i[m * n + j];
            const double* g = dZ + m * h;
            for (int64_t c = 0; c < h; ++c) w[c] += a * g[c];
        }
    }
    /* dW1_i[k][j] = sum_m X[m][k] dY_i[m][j] */
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < h; ++k) {
        double* w = dW1_i + k * n;
        for (int64_t j = 0; j < n; ++j) w[j] = 0.0;
        for (int64_t m = 0; m < T; ++m) {
            const double a = X[m * h + k];
            const double* g = dY_i + m * n;
            for (int64_t j = 0; j < n; ++j) w[j] += a * g[j];
        }
    }
    /* dX_i[m][k] = sum_j dY_i[m][j] W1_i[k][j] */
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < T; ++m) {
        for (int64_t k = 0; k < h; ++k) {
            double s = 0.0;
            for (int64_t j = 0; j < n; ++j) s += dY_i[m * n + j] * W1_i[k * n + j];
            dX_i[m * h + k] = s;
        }
    }
    /* db1_i[j] = sum_m dY_i[m][j] */
    if (db1_i) {
        for (int64_t j = 0; j < n; ++j) db1_i[j] = 0.0;
        for (int64_t m = 0; m < T; ++m)
            for (int64_t j = 0; j < n; ++j) db1_i[j] += dY_i[m * n + j];
    }
}

/* Backward of one linear shard Y = X W + b, the two gradients of the page
 * "Tensor Parallelism原理与实践" §3.1 written for a single shard (the column
 * layer's weight gradient X^T dL/dY and the input gradient dL/dY W^T) plus
 * the bias gradient (the chain rule through the bias):
 *   dX[m][k] = sum_j dY[m][j] W[k][j]
 *   dW[k][j] = sum_m X[m][k] dY[m][j]
 *   db[j]    = sum_m dY[m][j]              (db may be NULL)
 * Shapes: X [T,in]; W [in,out]; dY [T,out]; dX [T,in]; dW [in,out]; db [out]. */
ORACLE_API void oracle_linear_bwd(const double* X, const double* W, const double* dY,
                                  double* dX, double* dW, double* db, int64_t T, int64_t in,
                                  int64_t out)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < T; ++m) {
        for (int64_t k = 0; k < in; ++k) {
            double s = 0.0;
            for (int64_t j = 0; j < out; ++j) s += dY[m * out + j] * W[k * out + j];
            dX[m * in + k] = s;
        }
    }
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < in; ++k) {
        double* w = dW + k * out;
        for (int64_t j = 0; j < out; ++j) w[j] = 0.0;
        for (int64_t m = 0; m < T; ++m) {
            const double a = X[m * in + k];
            const double* g = dY + m * out;
            for (int64_t j = 0; j < out; ++j) w[j] += a * g[j];
        }
    }
    if (db) {
        for (int64_t j = 0; j < out; ++j) db[j] = 0.0;
        for (int64_t m = 0; m < T; ++m)
            for (int64_t j = 0; j < out; ++j) db[j] += dY[m * out + j];
    }
}

/* Stand-in for AllReduce(SUM) over t ranks [P4 §2.1, §2.2]:
 *   out[e] = parts[0][e] + parts[1][e] + ... + parts[t-1][e]   (rank order)
 * parts is [t][count] contiguous. */
ORACLE_API void oracle_shard_sum(const double* parts, double* out, int t, int64_t count)
{
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < count; ++e) {
        double s = 0.0;
        for (int r = 0; r < t; ++r) s += parts[(int64_t)r * count + e];
        out[e] = s;
    }
}

/* Stand-in for AllGather + concatenation along the last dimension in rank
 * order [P3 "PyTorch 实现示例"; P1 introduction]:
 *   out[m][r*cols + c] = parts[r][m][c]
 * parts is [t][rows][cols]; out is [rows][t*cols]. */
ORACLE_API void oracle_shard_concat(const double* parts, double* out, int t,
                                    int64_t rows, int64_t cols)
{
    for (int r = 0; r < t; ++r)
        for (int64_t m = 0; m < rows; ++m)
            memcpy(out + m * (t * cols) + (int64_t)r * cols,
                   parts + ((int64_t)r * rows + m) * cols, (size_t)cols * sizeof(double));
}

/* Sequence-parallel stand-ins.  Sequence parallelism extends tensor
 * parallelism by splitting the token dimension [P2 "延伸阅读", "相关概念推荐"];
 * the partial outputs are then combined by a ReduceScatter instead of an
 * AllReduce [P1 introduction]: rank `rank` keeps only its block of
 * rows / t tokens of the sum,
 *   out[m][c] = sum_{r=0}^{t-1} parts[r][rank * rows / t + m][c],
 * parts is [t][rows][cols], out is [rows / t][cols]; ranks added in order. */
ORACLE_API void oracle_reduce_scatter(const double* parts, double* out, int t, int64_t rows,
                                      int64_t cols, int rank)
{
    const int64_t rr = rows / t;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < rr; ++m)
        for (int64_t c = 0; c < cols; ++c) {
            double s = 0.0;
            for (int r = 0; r < t; ++r)
                s += parts[((int64_t)r * rows + (int64_t)rank * rr + m) * cols + c];
            out[m * cols + c] = s;
        }
}

/* Layer normalisation of whole rows (a token shard holds every hidden
 * column of its tokens, so the statistics need no exchange; the pages keep
 * normalisations unsplit [P1 introduction] or exchange the statistics when
 * the hidden dimension is split [P4 §4.2]):
 *   mu = (1/cols) sum_c x[m][c];  var = (1/cols) sum_c (x[m][c] - mu)^2
 *   y[m][c] = (x[m][c] - mu) / sqrt(var + eps) * gamma[c] + beta[c]
 * gamma == NULL means 1, beta == NULL means 0. */
ORACLE_API void oracle_layernorm(const double* x, const double* gamma, const double* beta,
                                 double* y, int64_t rows, int64_t cols, double eps)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < rows; ++m) {
        const double* xr = x + m * cols;
        double mu = 0.0;
        for (int64_t c = 0; c < cols; ++c) mu += xr[c];
        mu /= (double)cols;
        double var = 0.0;
        for (int64_t c = 0; c < cols; ++c) var += (xr[c] - mu) * (xr[c] - mu);
        var /= (double)cols;
        const double inv = 1.0 / sqrt(var + eps);
        for (int64_t c = 0; c < cols; ++c) {
            double v = (xr[c] - mu) * inv;
            if (gamma) v *= gamma[c];
            if (beta) v += beta[c];
            y[m * cols + c] = v;
        }
    }
}
