/*
 * tp_mlp.h - C ABI for one tensor-parallel rank's share of a transformer MLP
 * on AMD Instinct MI355X (gfx950).
 *
 * The layer is split the Megatron way: the first linear layer is column-
 * parallel (its weight is split by columns, every rank holds the whole input
 * X), the second is row-parallel (its weight is split by rows, its input is
 * the first layer's output shard), so the only exchanges are a sum of the
 * row layer's partial outputs in the forward and a sum of the input-gradient
 * partials in the backward.  On one GPU those exchanges are replaced by
 * tp_shard_reduce, which sums (or concatenates) the t shards held in HBM.
 *
 * Pages cited below:
 *   [P1] "PaddlePaddle张量并行：从原理到工业落地的深度解析", introduction
 *        (column split of the FFN weight, AllGather of the shards, input
 *        gradient aggregated by ReduceScatter / AllReduce).
 *   [P2] "张量并行是什么：2026 大模型训练核心原理与实战详解", section
 *        "核心工作机制：切分矩阵，协同计算" (column layer then row layer).
 *   [P3] "张量并行实战：从理论到PyTorch代码的完整落地指南", section
 *        "PyTorch 实现示例：自定义张量并行 Linear 层" (weight shard
 *        [in, out/t], x @ W + b, divisibility assert, rank-ordered concat).
 *   [P4] "Tensor Parallelism原理与实践：大模型训练的关键技术", §2.1 (block
 *        product, sum of partials), §3.1 (column and row backward), §4.2
 *        (split strategies per layer type: attention, layer normalisation).
 * Sequence parallelism (the token dimension split as well) is named by [P2]
 * section "延伸阅读" ("相关概念推荐") as the long-sequence extension of tensor
 * parallelism; its ReduceScatter is [P1]'s alternative to the AllReduce.
 *
 * Conventions shared by every entry point:
 *   - Matrices are dense, row-major and contiguous.  Weights are stored
 *     [in_features, out_features] and used as x @ W [P3].  Pointers are
 *     shard-local (the caller passes rank r's block, not the full matrix).
 *   - All pointers are device pointers (HBM, from hipMalloc or torch), owned
 *     by the caller.  The library never allocates or frees memory and keeps
 *     no mutable global state; calls are re-entrant.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Calls
 *     only enqueue work and return; nothing is synchronised.
 *   - Element types: TP_BF16 (bfloat16) or TP_F32 (float).  Products are
 *     accumulated in fp32 (MFMA).  bf16 results are rounded to nearest even.
 *   - `t` is the tensor-parallel degree (world size) and `rank` is in [0, t).
 *     rank only identifies which block the shard is; it is validated and
 *     does not change the arithmetic.
 *   - Dimensions: tokens >= 0 (0 is a no-op), every feature dimension (and
 *     the shard width out_features / t, in_features / t) must be a positive
 *     multiple of 8.  Each operand must be smaller than 2^31 bytes.
 *   - Pointers must be 16-byte aligned.  Optional pointers may be NULL.
 *   - No output may overlap an input or another output (the kernels read
 *     inputs while other workgroups write outputs, and the backward stages
 *     intermediate data in its outputs); the byte ranges the shape arguments
 *     give are compared and an overlap returns TP_ERR_OVERLAP.  The one
 *     exception is tp_layernorm with y == x exactly (in place).
 *   - Errors: arguments are validated before anything is enqueued; on any
 *     error nothing is launched and a negative tp_status is returned.  A
 *     failed launch returns TP_ERR_HIP (work enqueued earlier in the same
 *     call may already be on the stream).
 */
#ifndef TP_MLP_H
#define TP_MLP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef TP_API
#define TP_API __attribute__((visibility("default")))
#endif

typedef enum {
    TP_OK = 0,
    TP_ERR_NULL = -1,        /* a required pointer is NULL */
    TP_ERR_SHAPE = -2,       /* dimension negative, zero, not a multiple of 8, or too large */
    TP_ERR_INDIVISIBLE = -3, /* the split dimension is not divisible by t [P3 assert] */
    TP_ERR_RANK = -4,        /* t < 1 or rank outside [0, t) */
    TP_ERR_DTYPE = -5,       /* unsupported element-type combination */
    TP_ERR_ALIGN = -6,       /* a pointer is not 16-byte aligned */
    TP_ERR_HIP = -7,         /* the HIP runtime rejected a launch */
    TP_ERR_ARG = -8,         /* an enum argument is out of range */
    TP_ERR_OVERLAP = -9      /* an output overlaps an input or another output */
} tp_status;

typedef enum { TP_F32 = 0, TP_BF16 = 1 } tp_dtype;
typedef enum { TP_ACT_NONE = 0, TP_ACT_GELU_TANH = 1 } tp_act;
typedef enum { TP_REDUCE_SUM = 0, TP_REDUCE_CONCAT = 1, TP_REDUCE_CONCAT_TOKENS = 2 } tp_reduce_op;

/*
 * Column-parallel linear on one shard [P3; P4 §2.1; P1]:
 *   Y_i[m][j] = act( pre[m][j] ),  pre[m][j] = sum_k X[m][k] * W_i[k][j] + b_i[j]
 *   X   [tokens, in_features]              element type `dtype`
 *   W_i [in_features, out_features / t]    element type `dtype`
 *   b_i [out_features / t] or NULL (= 0)   element type `dtype`
 *   Y_i [tokens, out_features / t]         element type `out_dtype`
 *   pre_save [tokens, out_features / t] or NULL: receives the pre-activation
 *            (element type `dtype`), the value the backward's g'() needs;
 *            must be NULL with TP_ACT_NONE, where Y_i is the pre-activation
 *            itself (TP_ERR_ARG otherwise)
 * act: TP_ACT_NONE or TP_ACT_GELU_TANH, g(y) = 0.5 y (1 + tanh(sqrt(2/pi)
 * (y + 0.044715 y^3))).  dtype TP_F32 requires out_dtype TP_F32; dtype
 * TP_BF16 allows either.  out_features % t != 0 -> TP_ERR_INDIVISIBLE.
 */
TP_API int tp_column_linear(const void* X, const void* W_i, const void* b_i, void* Y_i,
                            void* pre_save, int64_t tokens, int64_t in_features,
                            int64_t out_features, int t, int rank, int dtype, int out_dtype,
                            int act, void* stream);

/*
 * Row-parallel linear on one shard, partial output without bias
 * [P2 "核心工作机制"; P4 §3.1 row parallel]:
 *   Z_i[m][c] = sum_j X_i[m][j] * W_i[j][c]
 *   X_i [tokens, in_features / t]          element type `dtype`
 *   W_i [in_features / t, out_features]    element type `dtype`
 *   Z_i [tokens, out_features]             element type `out_dtype`
 * The partials of all ranks add up to the unsharded product (tp_shard_reduce
 * with TP_REDUCE_SUM).  in_features % t != 0 -> TP_ERR_INDIVISIBLE.
 */
TP_API int tp_row_linear(const void* X_i, const void* W_i, void* Z_i,
                  int64_t tokens, int64_t in_features, int64_t out_features,
                  int t, int rank, int dtype, int out_dtype, void* stream);

/*
 * Forward of one MLP shard, column layer feeding the row layer with no
 * exchange in between [P2 "核心工作机制"; P4 §3.1].  Same kernels and order
 * as tp_column_linear(act = GeLU, out_dtype = dtype) followed by
 * tp_row_linear(out_dtype = fp32):
 *   Y_i = X W1_i + b1_i ;  H_i = g(Y_i) ;  Z_i = H_i W2_i
 *   X    [tokens, h]       W1_i [h, n]      b1_i [n] or NULL     W2_i [n, h]
 *   H_i  [tokens, n]  (required; it is an output and the row layer's input)
 *   Y_i_save [tokens, n] or NULL (pre-activation, kept for the backward)
 *   Z_i  [tokens, h]  fp32 partial output (sum over ranks = layer output)
 * with n = ffn / t.  X, W1_i, b1_i, W2_i, H_i, Y_i_save have element type
 * `dtype`; Z_i is always fp32.  ffn % t != 0 -> TP_ERR_INDIVISIBLE.
 */
TP_API int tp_mlp_shard_fwd(const void* X, const void* W1_i, const void* b1_i, const void* W2_i,
                     void* H_i, void* Y_i_save, void* Z_i,
                     int64_t tokens, int64_t h, int64_t ffn, int t, int rank,
                     int dtype, void* stream);

/*
 * Forward of every rank's MLP shard of one layer on this device, the t
 * shards' products batched into two launches (all column products, then all
 * row products) [P2 "核心工作机制"; P4 §2.1 (the layer output is the sum of
 * the t partials)].  For r = 0 .. t-1 it computes exactly what
 * tp_mlp_shard_fwd(rank = r) computes, bit for bit:
 *   Y_r = X W1[r] + b1[r] ;  H[r] = g(Y_r) ;  Z[r] = H[r] W2[r]
 * Buffers hold the shards stacked rank by rank (rank r's block at offset
 * r * <block size>), the layout tp_shard_reduce takes:
 *   X      [tokens, h]            shared by every rank
 *   W1     [t][h][n]    b1 [t][n] or NULL     W2 [t][n][h]
 *   H      [t][tokens][n]   (required; output and the row products' input)
 *   Y_save [t][tokens][n] or NULL (pre-activations, for the backward)
 *   Z      [t][tokens][h]   fp32 partial outputs; tp_shard_reduce with
 *                           TP_REDUCE_SUM adds them into the layer output
 * with n = ffn / t.  X, W1, b1, W2, H, Y_save have element type `dtype`.
 * Errors as tp_mlp_shard_fwd (t < 1 -> TP_ERR_RANK); each rank's block
 * must be smaller than 2^31 bytes.  Batching lets the tiles of all shards
 * share the GPU: a shard whose output is not a whole number of tile waves
 * (h = 8192, n = 3584: 304 tiles for 256 compute units) no longer leaves
 * most of a second wave idle.
 */
TP_API int tp_mlp_layer_fwd(const void* X, const void* W1, const void* b1, const void* W2,
                            void* H, void* Y_save, void* Z, int64_t tokens, int64_t h,
                            int64_t ffn, int t, int dtype, void* stream);

/*
 * Backward of one MLP shard from the full output gradient dZ (replicated on
 * every rank) and the forward's saved Y_i, H_i [P4 §3.1; P1]:
 *   dY_i  = (dZ W2_i^T) * g'(Y_i)      elementwise product
 *   dW2_i = H_i^T dZ
 *   dW1_i = X^T dY_i
 *   dX_i  = dY_i W1_i^T                this rank's share of dL/dX
 *   db1_i = sum over tokens of dY_i    (only if db1_i != NULL)
 *   inputs:  X [tokens,h], W1_i [h,n], W2_i [n,h], Y_i [tokens,n],
 *            H_i [tokens,n], dZ [tokens,h]         element type `dtype`
 *   outputs: dY_i [tokens,n] (element type `dtype`; also the input of the
 *            last two products), dW2_i [n,h], dW1_i [h,n], dX_i [tokens,h],
 *            db1_i [n] or NULL                     fp32
 * tokens == 0 is valid: the weight gradients are then written as zeros.
 * db1_i is summed in fp32 in a fixed order (run-to-run deterministic); its
 * summands are the dY product's fp32 results before rounding to `dtype` when
 * that product runs on the tile kernel and its per-256-row partials fit in
 * dW2_i (bf16, 256 <= tokens <= 256 h, n >= 192, h % 32 == 0), else the
 * stored dY_i.
 * dW2_i, dW1_i and dX_i also serve as scratch space during the call (partial
 * sums of db1_i; transposed copies of H_i and of dY_i or X) before they
 * receive their results, so no output may overlap an input.
 */
TP_API int tp_mlp_shard_bwd(const void* X, const void* W1_i, const void* W2_i,
                     const void* Y_i, const void* H_i, const void* dZ,
                     void* dY_i, void* dW2_i, void* dW1_i, void* dX_i, void* db1_i,
                     int64_t tokens, int64_t h, int64_t ffn, int t, int rank,
                     int dtype, void* stream);

/*
 * Backward of one linear shard Y = X W (+ b), from the gradient dY of its
 * output: the column layer's weight gradient and the input gradient of
 * [P4 §3.1] for a single shard, plus the bias gradient:
 *   dX = dY W^T    [tokens, in_features]           fp32
 *   dW = X^T dY    [in_features, out_features]     fp32
 *   db = sum over tokens of dY  [out_features]     fp32 (only if db != NULL)
 *   X [tokens, in_features], W [in_features, out_features],
 *   dY [tokens, out_features]                      element type `dtype`
 * The dimensions are the shard's own: for a column shard in_features = h and
 * out_features = n (its dX is this rank's partial, summed over ranks); for a
 * row shard in_features = n and out_features = h.  It serves every linear
 * layer of the path on its own (the attention projections, the column-only
 * layer).  dW and dX also serve as scratch during the call (partial sums of
 * db; a transposed copy of dY or X), so no output may overlap an input.
 * tokens == 0 writes a zero dW (and db).
 */
TP_API int tp_linear_bwd(const void* X, const void* W, const void* dY, void* dX, void* dW,
                         void* db, int64_t tokens, int64_t in_features, int64_t out_features,
                         int dtype, void* stream);

/*
 * Stand-in for the collective between ranks, over the t shards held on one
 * GPU.  parts is [t][tokens][cols], contiguous, element type in_dtype.
 *   TP_REDUCE_SUM    (AllReduce of row-parallel partials [P4 §2.1, §2.2]):
 *                    out[m][c] = parts[0][m][c] + ... + parts[t-1][m][c],
 *                    added in fp32 in rank order 0..t-1 (run-to-run
 *                    deterministic), out [tokens][cols] of type out_dtype.
 *   TP_REDUCE_CONCAT (AllGather + concat along the last dim [P3; P1]):
 *                    out[m][r*cols + c] = parts[r][m][c], out
 *                    [tokens][t*cols]; requires out_dtype == in_dtype.
 *   TP_REDUCE_CONCAT_TOKENS (AllGather of token shards before the column
 *                    layer under sequence parallelism [P2 "延伸阅读"]):
 *                    out[r*tokens + m][c] = parts[r][m][c], out
 *                    [t*tokens][cols]; requires out_dtype == in_dtype.
 * cols must be a positive multiple of 8; parts and out must not overlap.
 */
TP_API int tp_shard_reduce(const void* parts, void* out, int64_t tokens, int64_t cols, int t,
                    int op, int in_dtype, int out_dtype, void* stream);

/*
 * ReduceScatter over tokens, the sequence-parallel replacement of the
 * AllReduce of row-parallel partials [P1 introduction; P2 "延伸阅读"]: rank
 * `rank` keeps only its block of tokens / t rows of the sum,
 *   out[m][c] = parts[0][rank*tokens/t + m][c] + ... + parts[t-1][...][c],
 * added in fp32 in rank order 0..t-1.  parts is [t][tokens][cols] (type
 * in_dtype), out [tokens/t][cols] (type out_dtype).  tokens % t != 0 ->
 * TP_ERR_INDIVISIBLE; rank outside [0, t) -> TP_ERR_RANK; cols must be a
 * positive multiple of 8; parts and out must not overlap.
 */
TP_API int tp_shard_reduce_scatter(const void* parts, void* out, int64_t tokens, int64_t cols,
                                   int t, int rank, int in_dtype, int out_dtype, void* stream);

/*
 * Layer normalisation of whole rows, as a sequence-parallel rank applies it
 * to its token shard: each row holds every hidden column, so its statistics
 * need no exchange (the pages keep normalisations unsplit [P1 introduction]
 * or exchange statistics when the hidden dimension itself is split [P4
 * §4.2]):
 *   mu = mean_c x[m][c];  var = mean_c (x[m][c] - mu)^2  (biased)
 *   y[m][c] = (x[m][c] - mu) / sqrt(var + eps) * gamma[c] + beta[c]
 * Statistics in fp32 with a fixed reduction order (bitwise reproducible).
 * x [tokens][cols] of type in_dtype; y [tokens][cols] and gamma, beta [cols]
 * of type out_dtype; gamma NULL means 1, beta NULL means 0.  eps must be
 * finite and >= 0 (TP_ERR_ARG otherwise); cols a positive multiple of 8.
 * x and y may be the same buffer only when in_dtype == out_dtype.
 */
TP_API int tp_layernorm(const void* x, const void* gamma, const void* beta, void* y,
                        int64_t tokens, int64_t cols, float eps, int in_dtype, int out_dtype,
                        void* stream);

/*
 * ReduceScatter over tokens and the layer normalisation of the rank's rows,
 * in one pass: the sequence-parallel rank's path from the row-parallel
 * partials to its normalised token shard (ReduceScatter in place of the
 * AllReduce [P1 introduction; P2 "延伸阅读"], then the normalisation of whole
 * token rows, which needs no exchange of statistics [P1 introduction; P4
 * §4.2]):
 *   s[m][c] = parts[0][rank*tokens/t + m][c] + ... + parts[t-1][...][c]
 *             (fp32, rank order 0..t-1)
 *   y[m][c] = (s[m][c] - mu_m) / sqrt(var_m + eps) * gamma[c] + beta[c]
 * The result is bit for bit that of tp_shard_reduce_scatter with an fp32
 * output followed by tp_layernorm of that output, without writing or
 * re-reading s.  parts [t][tokens][cols] (in_dtype); y [tokens/t][cols] and
 * gamma, beta [cols] (out_dtype; gamma NULL means 1, beta NULL means 0).
 * Errors as for those two calls: tokens % t != 0 -> TP_ERR_INDIVISIBLE, rank
 * outside [0, t) -> TP_ERR_RANK, cols a positive multiple of 8, eps finite
 * and >= 0 (TP_ERR_ARG otherwise); y must not overlap parts, gamma or beta.
 */
TP_API int tp_shard_reduce_scatter_layernorm(const void* parts, const void* gamma,
                                             const void* beta, void* y, int64_t tokens,
                                             int64_t cols, int t, int rank, float eps,
                                             int in_dtype, int out_dtype, void* stream);

/* Static description of a status code (never NULL). */
TP_API const char* tp_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* TP_MLP_H */
