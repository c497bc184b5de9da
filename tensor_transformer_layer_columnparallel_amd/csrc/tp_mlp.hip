// C entry points of libtpmlp: argument validation, then kernel launches on the
// caller's stream.  The declarations, with the meaning of every argument and
// the pages each operation follows, are in include/tp_mlp.h.
#include "tp_mlp.h"

#include "common.h"
#include "kernels.h"

using namespace tpmlp;

namespace {

constexpr int64_t kMaxOperandBytes = (int64_t(1) << 31) - 1;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elt_size(int dtype) { return dtype == TP_F32 ? 4 : 2; }

bool valid_dtype(int d) { return d == TP_F32 || d == TP_BF16; }

Elt to_elt(int d) { return d == TP_F32 ? Elt::F32 : Elt::BF16; }

// A feature dimension: positive multiple of 8.
bool feature_dim_ok(int64_t d) { return d > 0 && d % 8 == 0; }

bool fits(int64_t rows, int64_t cols, int bytes)
{
    if (rows < 0 || cols < 0) return false;
    if (rows == 0 || cols == 0) return true;
    return rows <= kMaxOperandBytes / cols / bytes;
}

int check_ptrs(std::initializer_list<const void*> required,
               std::initializer_list<const void*> optional)
{
    for (const void* p : required)
        if (!p) return TP_ERR_NULL;
    for (const void* p : required)
        if (!aligned16(p)) return TP_ERR_ALIGN;
    for (const void* p : optional)
        if (p && !aligned16(p)) return TP_ERR_ALIGN;
    return TP_OK;
}

int check_split(int64_t full, int t, int rank, int64_t* local)
{
    if (t < 1 || rank < 0 || rank >= t) return TP_ERR_RANK;
    if (!feature_dim_ok(full)) return TP_ERR_SHAPE;
    if (full % t != 0) return TP_ERR_INDIVISIBLE;
    *local = full / t;
    if (!feature_dim_ok(*local)) return TP_ERR_SHAPE;
    return TP_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? TP_OK : TP_ERR_HIP; }

// A byte range [p, p + bytes) that an entry point reads or writes.
struct Region {
    const void* p;
    int64_t bytes;
};

// a * b * c * es, saturating at INT64_MAX (shapes here are non-negative).
int64_t nbytes(int64_t a, int64_t b, int64_t c, int64_t es)
{
    int64_t r = es;
    for (int64_t d : {a, b, c}) {
        if (d <= 0) return 0;
        if (r > INT64_MAX / d) return INT64_MAX;
        r *= d;
    }
    return r;
}

bool overlap(const Region& a, const Region& b)
{
    if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    const uintptr_t a1 = a0 + (uintptr_t)a.bytes < a0 ? UINTPTR_MAX : a0 + (uintptr_t)a.bytes;
    const uintptr_t b1 = b0 + (uintptr_t)b.bytes < b0 ? UINTPTR_MAX : b0 + (uintptr_t)b.bytes;
    return a0 < b1 && b0 < a1;
}

// TP_ERR_OVERLAP if an output overlaps an input or another output.
int check_overlap(std::initializer_list<Region> outs, std::initializer_list<Region> ins)
{
    for (auto o = outs.begin(); o != outs.end(); ++o) {
        for (const Region& i : ins)
            if (overlap(*o, i)) return TP_ERR_OVERLAP;
        for (auto o2 = o + 1; o2 != outs.end(); ++o2)
            if (overlap(*o, *o2)) return TP_ERR_OVERLAP;
    }
    return TP_OK;
}

// The weight-gradient products x^T dy read both operands M/N-contiguous,
// which the tile kernel can only do with transposing LDS reads of both.  With
// bf16 operands, a token count that whole 32-deep slabs cover and room for
// H_i^T (n x T bf16) in the fp32 dW1_i (h x n), one activation per product
// is transposed first (an HBM-bound pass) and the products run with a
// K-contiguous first operand: H_i^T dZ, and dY_i^T X stored transposed (or
// X^T dY_i where dY_i^T does not fit in dX_i).
bool use_transposed_operands(int64_t tokens, int64_t h, int64_t n, Elt e)
{
    if (e != Elt::BF16 || tokens == 0 || tokens % 32 != 0) return false;
    if (2 * tokens > 4 * h) return false;   // H_i^T must fit in dW1_i
    GemmArgs a{};
    a.M = n; a.N = h; a.K = tokens;
    GemmArgs b{};
    b.M = h; b.N = n; b.K = tokens;
    return gemm_ring_supported(a, Layout::NN) && gemm_ring_supported(b, Layout::NN);
}

// True when a product of this shape (`batch` of them in one launch) runs on
// the tile kernel.
bool ring_path(int64_t M, int64_t N, int64_t K, Elt elt, Layout layout, int64_t batch = 1,
               int64_t lda = 0, int64_t ldb = 0)
{
    GemmArgs p{};
    p.M = M; p.N = N; p.K = K;
    p.batch = batch;
    p.lda = lda; p.ldb = ldb;
    return elt == Elt::BF16 && M > 0 && N > 0 && gemm_ring_supported(p, layout);
}

// `batch` products of one shape with operands at the given element strides
// (A, B, C, bias, save), one launch on the tile kernel.
struct Batch {
    int64_t count = 1, sA = 0, sB = 0, sC = 0, sBias = 0, sSave = 0;
    int64_t lda = 0, ldb = 0;   // row strides when not packed (tile kernel only)
};

// Split over K of the x W^T product dX[T][k] = dY[T][n] W[k][n]^T when its
// output is too few 256 x 192 tiles to fill the GPU (the attention output
// projection's dX: [2048, 1536], K = 12288, 64 tiles): s products over K
// ranges of n / s, whose fp32 partials ([s][T][k]) must fit in `scratch_bytes`,
// are summed in order afterwards.  Returns s (1: no split).
int64_t dx_split(int64_t tokens, int64_t k, int64_t n, Elt e, int64_t scratch_bytes)
{
    if (e != Elt::BF16 || tokens == 0) return 1;
    const int64_t tiles = ((tokens + 255) / 256) * ((k + 191) / 192);
    int64_t s = 1;
    while (s < 8 && tiles * s * 2 <= 256 && n % (32 * s * 2) == 0 &&
           s * 2 * tokens * k * 4 <= scratch_bytes &&
           ring_path(tokens, k, n / (s * 2), e, Layout::NT, s * 2, n, n))
        s *= 2;
    return s;
}

// colsum (DGelu on the tile kernel only): per-256-row-block column sums of C.
hipError_t run_gemm(const void* A, const void* B, void* C, const void* bias, const void* aux,
                    void* save, int64_t M, int64_t N, int64_t K, Elt elt, Layout layout, Epi epi,
                    Elt out, hipStream_t stream, float* colsum = nullptr,
                    const Batch& batch = Batch{})
{
    if (M == 0 || N == 0 || batch.count == 0) return hipSuccess;
    GemmArgs p{A, B, C, bias, aux, save, M, N, K, colsum};
    p.batch = batch.count;
    p.sA = batch.sA; p.sB = batch.sB; p.sC = batch.sC;
    p.sBias = batch.sBias; p.sSave = batch.sSave;
    p.lda = batch.lda; p.ldb = batch.ldb;
    if (ring_path(M, N, K, elt, layout, batch.count, batch.lda, batch.ldb))
        return gemm_ring(p, layout, epi, out, stream);
    return gemm_simple(p, elt, layout, epi, out, stream);
}

}  // namespace

extern "C" {

const char* tp_status_string(int status)
{
    switch (status) {
    case TP_OK: return "ok";
    case TP_ERR_NULL: return "a required pointer is NULL";
    case TP_ERR_SHAPE: return "a dimension is negative, zero, not a multiple of 8, or too large";
    case TP_ERR_INDIVISIBLE: return "the split dimension is not divisible by t";
    case TP_ERR_RANK: return "t < 1 or rank outside [0, t)";
    case TP_ERR_DTYPE: return "unsupported element-type combination";
    case TP_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case TP_ERR_HIP: return "the HIP runtime rejected a launch";
    case TP_ERR_ARG: return "an enum argument is out of range";
    case TP_ERR_OVERLAP: return "an output overlaps an input or another output";
    default: return "unknown status";
    }
}

int tp_column_linear(const void* X, const void* W_i, const void* b_i, void* Y_i,
                     void* pre_save, int64_t tokens, int64_t in_features, int64_t out_features,
                     int t, int rank, int dtype, int out_dtype, int act, void* stream)
{
    if (!valid_dtype(dtype) || !valid_dtype(out_dtype)) return TP_ERR_DTYPE;
    if (dtype == TP_F32 && out_dtype != TP_F32) return TP_ERR_DTYPE;
    if (act != TP_ACT_NONE && act != TP_ACT_GELU_TANH) return TP_ERR_ARG;
    int st = check_ptrs({X, W_i, Y_i}, {b_i, pre_save});
    if (st) return st;
    int64_t n = 0;
    if ((st = check_split(out_features, t, rank, &n))) return st;
    if (tokens < 0 || !feature_dim_ok(in_features)) return TP_ERR_SHAPE;
    const int es = elt_size(dtype);
    if (!fits(tokens, in_features, es) || !fits(in_features, n, es) ||
        !fits(tokens, n, elt_size(out_dtype)) || !fits(tokens, n, es))
        return TP_ERR_SHAPE;
    // Without an activation the output is the pre-activation itself.
    const Epi epi = act == TP_ACT_GELU_TANH ? Epi::BiasGelu : Epi::Bias;
    if (epi == Epi::Bias && pre_save) return TP_ERR_ARG;
    if ((st = check_overlap({{Y_i, nbytes(tokens, n, 1, elt_size(out_dtype))},
                             {pre_save, nbytes(tokens, n, 1, es)}},
                            {{X, nbytes(tokens, in_features, 1, es)},
                             {W_i, nbytes(in_features, n, 1, es)}, {b_i, nbytes(n, 1, 1, es)}})))
        return st;
    return status_of(run_gemm(X, W_i, Y_i, b_i, nullptr, pre_save, tokens, n, in_features,
                              to_elt(dtype), Layout::NN, epi, to_elt(out_dtype),
                              static_cast<hipStream_t>(stream)));
}

int tp_row_linear(const void* X_i, const void* W_i, void* Z_i, int64_t tokens,
                  int64_t in_features, int64_t out_features, int t, int rank, int dtype,
                  int out_dtype, void* stream)
{
    if (!valid_dtype(dtype) || !valid_dtype(out_dtype)) return TP_ERR_DTYPE;
    if (dtype == TP_F32 && out_dtype != TP_F32) return TP_ERR_DTYPE;
    int st = check_ptrs({X_i, W_i, Z_i}, {});
    if (st) return st;
    int64_t k = 0;
    if ((st = check_split(in_features, t, rank, &k))) return st;
    if (tokens < 0 || !feature_dim_ok(out_features)) return TP_ERR_SHAPE;
    const int es = elt_size(dtype);
    if (!fits(tokens, k, es) || !fits(k, out_features, es) ||
        !fits(tokens, out_features, elt_size(out_dtype)))
        return TP_ERR_SHAPE;
    if ((st = check_overlap({{Z_i, nbytes(tokens, out_features, 1, elt_size(out_dtype))}},
                            {{X_i, nbytes(tokens, k, 1, es)},
                             {W_i, nbytes(k, out_features, 1, es)}})))
        return st;
    return status_of(run_gemm(X_i, W_i, Z_i, nullptr, nullptr, nullptr, tokens, out_features, k,
                              to_elt(dtype), Layout::NN, Epi::Store, to_elt(out_dtype),
                              static_cast<hipStream_t>(stream)));
}

int tp_mlp_shard_fwd(const void* X, const void* W1_i, const void* b1_i, const void* W2_i,
                     void* H_i, void* Y_i_save, void* Z_i, int64_t tokens, int64_t h,
                     int64_t ffn, int t, int rank, int dtype, void* stream)
{
    if (!valid_dtype(dtype)) return TP_ERR_DTYPE;
    int st = check_ptrs({X, W1_i, W2_i, H_i, Z_i}, {b1_i, Y_i_save});
    if (st) return st;
    int64_t n = 0;
    if ((st = check_split(ffn, t, rank, &n))) return st;
    if (tokens < 0 || !feature_dim_ok(h)) return TP_ERR_SHAPE;
    const int es = elt_size(dtype);
    if (!fits(tokens, h, es) || !fits(h, n, es) || !fits(tokens, n, es) || !fits(tokens, h, 4))
        return TP_ERR_SHAPE;
    if ((st = check_overlap({{H_i, nbytes(tokens, n, 1, es)}, {Y_i_save, nbytes(tokens, n, 1, es)},
                             {Z_i, nbytes(tokens, h, 1, 4)}},
                            {{X, nbytes(tokens, h, 1, es)}, {W1_i, nbytes(h, n, 1, es)},
                             {b1_i, nbytes(n, 1, 1, es)}, {W2_i, nbytes(n, h, 1, es)}})))
        return st;
    const Elt e = to_elt(dtype);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err = run_gemm(X, W1_i, H_i, b1_i, nullptr, Y_i_save, tokens, n, h, e, Layout::NN,
                              Epi::BiasGelu, e, s);
    if (err != hipSuccess) return TP_ERR_HIP;
    return status_of(run_gemm(H_i, W2_i, Z_i, nullptr, nullptr, nullptr, tokens, h, n, e,
                              Layout::NN, Epi::Store, Elt::F32, s));
}

int tp_mlp_layer_fwd(const void* X, const void* W1, const void* b1, const void* W2, void* H,
                     void* Y_save, void* Z, int64_t tokens, int64_t h, int64_t ffn, int t,
                     int dtype, void* stream)
{
    if (!valid_dtype(dtype)) return TP_ERR_DTYPE;
    int st = check_ptrs({X, W1, W2, H, Z}, {b1, Y_save});
    if (st) return st;
    int64_t n = 0;
    if ((st = check_split(ffn, t, 0, &n))) return st;
    if (tokens < 0 || !feature_dim_ok(h)) return TP_ERR_SHAPE;
    const int es = elt_size(dtype);
    if (!fits(tokens, h, es) || !fits(h, n, es) || !fits(tokens, n, es) || !fits(tokens, h, 4))
        return TP_ERR_SHAPE;
    if ((st = check_overlap({{H, nbytes(t, tokens, n, es)}, {Y_save, nbytes(t, tokens, n, es)},
                             {Z, nbytes(t, tokens, h, 4)}},
                            {{X, nbytes(tokens, h, 1, es)}, {W1, nbytes(t, h, n, es)},
                             {b1, nbytes(t, n, 1, es)}, {W2, nbytes(t, n, h, es)}})))
        return st;
    const Elt e = to_elt(dtype);
    hipStream_t s = static_cast<hipStream_t>(stream);
    Batch col;
    col.count = t;
    col.sB = h * n;          // W1[r]
    col.sC = tokens * n;     // H[r]
    col.sBias = n;           // b1[r]
    col.sSave = tokens * n;  // Y_save[r]
    hipError_t err = run_gemm(X, W1, H, b1, nullptr, Y_save, tokens, n, h, e, Layout::NN,
                              Epi::BiasGelu, e, s, nullptr, col);
    if (err != hipSuccess) return TP_ERR_HIP;
    Batch row;
    row.count = t;
    row.sA = tokens * n;     // H[r]
    row.sB = n * h;          // W2[r]
    row.sC = tokens * h;     // Z[r]
    return status_of(run_gemm(H, W2, Z, nullptr, nullptr, nullptr, tokens, h, n, e, Layout::NN,
                              Epi::Store, Elt::F32, s, nullptr, row));
}

int tp_mlp_shard_bwd(const void* X, const void* W1_i, const void* W2_i, const void* Y_i,
                     const void* H_i, const void* dZ, void* dY_i, void* dW2_i, void* dW1_i,
                     void* dX_i, void* db1_i, int64_t tokens, int64_t h, int64_t ffn, int t,
                     int rank, int dtype, void* stream)
{
    if (!valid_dtype(dtype)) return TP_ERR_DTYPE;
    int st = check_ptrs({X, W1_i, W2_i, Y_i, H_i, dZ, dY_i, dW2_i, dW1_i, dX_i}, {db1_i});
    if (st) return st;
    int64_t n = 0;
    if ((st = check_split(ffn, t, rank, &n))) return st;
    if (tokens < 0 || !feature_dim_ok(h)) return TP_ERR_SHAPE;
    const int es = elt_size(dtype);
    if (!fits(tokens, h, es) || !fits(h, n, es) || !fits(tokens, n, es) || !fits(tokens, h, 4) ||
        !fits(h, n, 4))
        return TP_ERR_SHAPE;
    if ((st = check_overlap({{dY_i, nbytes(tokens, n, 1, es)}, {dW2_i, nbytes(n, h, 1, 4)},
                             {dW1_i, nbytes(h, n, 1, 4)}, {dX_i, nbytes(tokens, h, 1, 4)},
                             {db1_i, nbytes(n, 1, 1, 4)}},
                            {{X, nbytes(tokens, h, 1, es)}, {W1_i, nbytes(h, n, 1, es)},
                             {W2_i, nbytes(n, h, 1, es)}, {Y_i, nbytes(tokens, n, 1, es)},
                             {H_i, nbytes(tokens, n, 1, es)}, {dZ, nbytes(tokens, h, 1, es)}})))
        return st;
    const Elt e = to_elt(dtype);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err;
    // dY_i = (dZ W2_i^T) * g'(Y_i): W2_i [n][h] is the K-contiguous [N][K] operand.
    // db1_i = column sums of dY_i.  On the tile kernel the product's epilogue
    // sums each 256-row block of its fp32 results and one pass adds the
    // blocks in order; otherwise a column-sum pass reads dY_i back.  Either
    // way dW2_i (written only afterwards) holds the partial sums.
    const int64_t row_blocks = (tokens + kGemmRingTileRows - 1) / kGemmRingTileRows;
    float* colsum = nullptr;
    if (db1_i && ring_path(tokens, n, h, e, Layout::NT) && row_blocks <= h)
        colsum = static_cast<float*>(dW2_i);
    if ((err = run_gemm(dZ, W2_i, dY_i, nullptr, Y_i, nullptr, tokens, n, h, e, Layout::NT,
                        Epi::DGelu, e, s, colsum)) != hipSuccess)
        return TP_ERR_HIP;
    // With the transposed operands the blocks' partials are added up in the
    // launch of the first transpose (both read and write disjoint memory,
    // and the partials are in dW2_i until its product); otherwise by their
    // own pass here.
    const bool transposed = use_transposed_operands(tokens, h, n, e);
    if (colsum && !transposed) {
        if ((err = column_finish(colsum, static_cast<float*>(db1_i), row_blocks, n, s)) !=
            hipSuccess)
            return TP_ERR_HIP;
    } else if (!colsum && db1_i &&
               (err = column_sum(dY_i, static_cast<float*>(db1_i), tokens, n, e, dW2_i,
                                 n * h * 4, s)) != hipSuccess) {
        return TP_ERR_HIP;
    }
    if (transposed) {
        // The weight gradients as products with a K-contiguous first operand.
        // dW2_i = (H_i^T) dZ, with H_i^T [n][T] staged in dW1_i's memory
        // (written only afterwards).
        if ((err = transpose16(H_i, dW1_i, tokens, n, s, colsum, static_cast<float*>(db1_i),
                               colsum ? row_blocks : 0, colsum ? n : 0)) != hipSuccess ||
            (err = run_gemm(dW1_i, dZ, dW2_i, nullptr, nullptr, nullptr, n, h, tokens, e,
                            Layout::NN, Epi::Store, Elt::F32, s)) != hipSuccess)
            return TP_ERR_HIP;
        if (n <= 2 * h) {
            // dW1_i^T = (dY_i^T) X, stored transposed into dW1_i: dY_i^T
            // [n][T] (half the bytes of X^T when n = h / 2) is staged in
            // dX_i's memory (written last).
            if ((err = transpose16(dY_i, dX_i, tokens, n, s)) != hipSuccess ||
                (err = run_gemm(dX_i, X, dW1_i, nullptr, nullptr, nullptr, n, h, tokens, e,
                                Layout::NN, Epi::StoreT, Elt::F32, s)) != hipSuccess)
                return TP_ERR_HIP;
        } else {
            // dW1_i = (X^T) dY_i with X^T [h][T] staged in dX_i's memory.
            if ((err = transpose16(X, dX_i, tokens, h, s)) != hipSuccess ||
                (err = run_gemm(dX_i, dY_i, dW1_i, nullptr, nullptr, nullptr, h, n, tokens, e,
                                Layout::NN, Epi::Store, Elt::F32, s)) != hipSuccess)
                return TP_ERR_HIP;
        }
    } else {
        // dW2_i = H_i^T dZ: H_i [T][n] is [K][M], dZ [T][h] is [K][N].
        if ((err = run_gemm(H_i, dZ, dW2_i, nullptr, nullptr, nullptr, n, h, tokens, e,
                            Layout::TN, Epi::Store, Elt::F32, s)) != hipSuccess)
            return TP_ERR_HIP;
        // dW1_i = X^T dY_i: X [T][h] is [K][M], dY_i [T][n] is [K][N].
        if ((err = run_gemm(X, dY_i, dW1_i, nullptr, nullptr, nullptr, h, n, tokens, e,
                            Layout::TN, Epi::Store, Elt::F32, s)) != hipSuccess)
            return TP_ERR_HIP;
    }
    // dX_i = dY_i W1_i^T: W1_i [h][n] is the K-contiguous [N][K] operand.
    if ((err = run_gemm(dY_i, W1_i, dX_i, nullptr, nullptr, nullptr, tokens, h, n, e, Layout::NT,
                        Epi::Store, Elt::F32, s)) != hipSuccess)
        return TP_ERR_HIP;
    return TP_OK;
}

int tp_linear_bwd(const void* X, const void* W, const void* dY, void* dX, void* dW, void* db,
                  int64_t tokens, int64_t in_features, int64_t out_features, int dtype,
                  void* stream)
{
    if (!valid_dtype(dtype)) return TP_ERR_DTYPE;
    int st = check_ptrs({X, W, dY, dX, dW}, {db});
    if (st) return st;
    if (tokens < 0 || !feature_dim_ok(in_features) || !feature_dim_ok(out_features))
        return TP_ERR_SHAPE;
    const int64_t k = in_features, n = out_features;
    const int es = elt_size(dtype);
    if (!fits(tokens, k, es) || !fits(k, n, es) || !fits(tokens, n, es) || !fits(tokens, k, 4) ||
        !fits(k, n, 4))
        return TP_ERR_SHAPE;
    if ((st = check_overlap({{dX, nbytes(tokens, k, 1, 4)}, {dW, nbytes(k, n, 1, 4)},
                             {db, nbytes(n, 1, 1, 4)}},
                            {{X, nbytes(tokens, k, 1, es)}, {W, nbytes(k, n, 1, es)},
                             {dY, nbytes(tokens, n, 1, es)}})))
        return st;
    const Elt e = to_elt(dtype);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t err;
    // db = column sums of dY, with dW (written only afterwards) as scratch for
    // the partial sums.
    if (db && (err = column_sum(dY, static_cast<float*>(db), tokens, n, e, dW, k * n * 4, s)) !=
                  hipSuccess)
        return TP_ERR_HIP;
    // dX split over K: the partials go to dW's memory (written afterwards),
    // are summed in order into dX, and dW is then computed with the
    // transposed reads of both operands (no memory is left to stage a
    // transposed copy).
    const int64_t split = dx_split(tokens, k, n, e, k * n * 4);
    if (split > 1) {
        Batch b;
        b.count = split;
        b.sA = n / split;        // dY columns of K range j
        b.sB = n / split;        // W columns of K range j
        b.sC = tokens * k;       // partial j
        b.lda = n;
        b.ldb = n;
        if ((err = run_gemm(dY, W, dW, nullptr, nullptr, nullptr, tokens, k, n / split, e,
                            Layout::NT, Epi::Store, Elt::F32, s, nullptr, b)) != hipSuccess ||
            (err = shard_sum(dW, dX, tokens * k, tokens * k, (int)split, Elt::F32, Elt::F32,
                             s)) != hipSuccess)
            return TP_ERR_HIP;
        return status_of(run_gemm(X, dY, dW, nullptr, nullptr, nullptr, k, n, tokens, e,
                                  Layout::TN, Epi::Store, Elt::F32, s));
    }
    // dW = X^T dY.  Both operands are M/N-contiguous; with bf16 and whole
    // 32-deep slabs of tokens the smaller activation is transposed into dX's
    // memory (written last) first, so that the tile kernel reads a
    // K-contiguous first operand: dW^T = (dY^T) X stored transposed when
    // out <= in, else (X^T) dY.
    const bool slabs = e == Elt::BF16 && tokens > 0 && tokens % 32 == 0;
    if (slabs && n <= k && ring_path(n, k, tokens, e, Layout::NN)) {
        if ((err = transpose16(dY, dX, tokens, n, s)) != hipSuccess ||
            (err = run_gemm(dX, X, dW, nullptr, nullptr, nullptr, n, k, tokens, e, Layout::NN,
                            Epi::StoreT, Elt::F32, s)) != hipSuccess)
            return TP_ERR_HIP;
    } else if (slabs && ring_path(k, n, tokens, e, Layout::NN)) {
        if ((err = transpose16(X, dX, tokens, k, s)) != hipSuccess ||
            (err = run_gemm(dX, dY, dW, nullptr, nullptr, nullptr, k, n, tokens, e, Layout::NN,
                            Epi::Store, Elt::F32, s)) != hipSuccess)
            return TP_ERR_HIP;
    } else if ((err = run_gemm(X, dY, dW, nullptr, nullptr, nullptr, k, n, tokens, e, Layout::TN,
                               Epi::Store, Elt::F32, s)) != hipSuccess) {
        return TP_ERR_HIP;
    }
    // dX = dY W^T: W [k][n] is the K-contiguous [N][K] operand.
    return status_of(run_gemm(dY, W, dX, nullptr, nullptr, nullptr, tokens, k, n, e, Layout::NT,
                              Epi::Store, Elt::F32, s));
}

int tp_shard_reduce(const void* parts, void* out, int64_t tokens, int64_t cols, int t, int op,
                    int in_dtype, int out_dtype, void* stream)
{
    if (op != TP_REDUCE_SUM && op != TP_REDUCE_CONCAT && op != TP_REDUCE_CONCAT_TOKENS)
        return TP_ERR_ARG;
    if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return TP_ERR_DTYPE;
    if (op != TP_REDUCE_SUM && in_dtype != out_dtype) return TP_ERR_DTYPE;
    int st = check_ptrs({parts, out}, {});
    if (st) return st;
    if (t < 1) return TP_ERR_RANK;
    if (tokens < 0 || !feature_dim_ok(cols)) return TP_ERR_SHAPE;
    const int64_t out_rows = op == TP_REDUCE_SUM ? 1 : t;   // CONCAT: t blocks of tokens x cols
    if ((st = check_overlap({{out, nbytes(out_rows, tokens, cols, elt_size(out_dtype))}},
                            {{parts, nbytes(t, tokens, cols, elt_size(in_dtype))}})))
        return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t count = tokens * cols;
    if (op == TP_REDUCE_SUM)
        return status_of(shard_sum(parts, out, count, count, t, to_elt(in_dtype),
                                   to_elt(out_dtype), s));
    if (op == TP_REDUCE_CONCAT_TOKENS)   // [t][tokens][cols] is already [t*tokens][cols]
        return status_of(shard_sum(parts, out, (int64_t)t * count, 0, 1, to_elt(in_dtype),
                                   to_elt(out_dtype), s));
    return status_of(shard_concat(parts, out, tokens, cols, t, to_elt(in_dtype), s));
}

int tp_shard_reduce_scatter(const void* parts, void* out, int64_t tokens, int64_t cols, int t,
                            int rank, int in_dtype, int out_dtype, void* stream)
{
    if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return TP_ERR_DTYPE;
    int st = check_ptrs({parts, out}, {});
    if (st) return st;
    if (t < 1 || rank < 0 || rank >= t) return TP_ERR_RANK;
    if (tokens < 0 || !feature_dim_ok(cols)) return TP_ERR_SHAPE;
    if (tokens % t != 0) return TP_ERR_INDIVISIBLE;
    const int64_t rows = tokens / t;
    if ((st = check_overlap({{out, nbytes(rows, cols, 1, elt_size(out_dtype))}},
                            {{parts, nbytes(t, tokens, cols, elt_size(in_dtype))}})))
        return st;
    const char* base = static_cast<const char*>(parts) + rank * rows * cols * elt_size(in_dtype);
    return status_of(shard_sum(base, out, rows * cols, tokens * cols, t, to_elt(in_dtype),
                               to_elt(out_dtype), static_cast<hipStream_t>(stream)));
}

int tp_shard_reduce_scatter_layernorm(const void* parts, const void* gamma, const void* beta,
                                      void* y, int64_t tokens, int64_t cols, int t, int rank,
                                      float eps, int in_dtype, int out_dtype, void* stream)
{
    if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return TP_ERR_DTYPE;
    int st = check_ptrs({parts, y}, {gamma, beta});
    if (st) return st;
    if (t < 1 || rank < 0 || rank >= t) return TP_ERR_RANK;
    if (tokens < 0 || !feature_dim_ok(cols)) return TP_ERR_SHAPE;
    if (tokens % t != 0) return TP_ERR_INDIVISIBLE;
    if (!(eps >= 0.0f) || eps == INFINITY) return TP_ERR_ARG;
    const int64_t rows = tokens / t;
    if ((st = check_overlap({{y, nbytes(rows, cols, 1, elt_size(out_dtype))}},
                            {{parts, nbytes(t, tokens, cols, elt_size(in_dtype))},
                             {gamma, nbytes(cols, 1, 1, elt_size(out_dtype))},
                             {beta, nbytes(cols, 1, 1, elt_size(out_dtype))}})))
        return st;
    const char* base = static_cast<const char*>(parts) + rank * rows * cols * elt_size(in_dtype);
    return status_of(sum_layernorm(base, tokens * cols, t, gamma, beta, y, rows, cols, eps,
                                   to_elt(in_dtype), to_elt(out_dtype),
                                   static_cast<hipStream_t>(stream)));
}

int tp_layernorm(const void* x, const void* gamma, const void* beta, void* y, int64_t tokens,
                 int64_t cols, float eps, int in_dtype, int out_dtype, void* stream)
{
    if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype)) return TP_ERR_DTYPE;
    int st = check_ptrs({x, y}, {gamma, beta});
    if (st) return st;
    if (tokens < 0 || !feature_dim_ok(cols)) return TP_ERR_SHAPE;
    if (!(eps >= 0.0f) || eps == INFINITY) return TP_ERR_ARG;
    if (x == y && in_dtype != out_dtype) return TP_ERR_ARG;
    if (!fits(tokens, cols, 4)) return TP_ERR_SHAPE;
    // y == x (in place) is allowed; any other overlap is not.
    if ((st = check_overlap({{y, nbytes(tokens, cols, 1, elt_size(out_dtype))}},
                            {{x == y ? nullptr : x, nbytes(tokens, cols, 1, elt_size(in_dtype))},
                             {gamma, nbytes(cols, 1, 1, elt_size(out_dtype))},
                             {beta, nbytes(cols, 1, 1, elt_size(out_dtype))}})))
        return st;
    return status_of(layernorm(x, gamma, beta, y, tokens, cols, eps, to_elt(in_dtype),
                               to_elt(out_dtype), static_cast<hipStream_t>(stream)));
}

}  // extern "C"
