// Shared device-side definitions of libtpmlp (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpmlp {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

#define TP_LDS __attribute__((address_space(3)))

// Element type tags used as template parameters.
enum class Elt { F32 = 0, BF16 = 1 };

// Epilogue applied to the fp32 accumulator tile.
enum class Epi {
    Store = 0,      // C = acc
    Bias = 1,       // C = acc + bias[col]
    BiasGelu = 2,   // Y = acc + bias[col] (optionally saved), C = g(Y)
    DGelu = 3,      // C = acc * g'(aux[row][col])
    StoreT = 4,     // C^T = acc: C is [N][M] (fp32 results only)
};

template <Elt E> struct EltType;
template <> struct EltType<Elt::F32> { typedef float type; };
template <> struct EltType<Elt::BF16> { typedef bf16 type; };

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
// fp32 -> bf16, round to nearest even (the hardware conversion on gfx950).
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

// Launch descriptor of one GEMM C[M,N] = op(A)[M,K] * op(B)[K,N].
//   a_kmajor: A stored [M][K] (K contiguous), else [K][M] (M contiguous)
//   b_kmajor: B stored [N][K] (K contiguous), else [K][N] (N contiguous)
struct GemmArgs {
    const void* A;
    const void* B;
    void* C;
    const void* bias;   // [N], element type of A/B; may be null
    const void* aux;    // DGelu: pre-activation [M][N]; BiasGelu: unused
    void* save;         // BiasGelu: pre-activation output [M][N]; may be null
    int64_t M, N, K;
    // DGelu, tile kernel only: column sums of C over each 256-row block of
    // tiles, fp32 [ceil(M / 256)][N], summed in a fixed order; may be null.
    float* colsum;
    // `batch` independent products of this shape in one launch, product b
    // reading A + b sA, B + b sB (and bias + b sBias) and writing C + b sC
    // (and save + b sSave); strides in elements.  Store, Bias and BiasGelu
    // epilogues only.
    int64_t batch = 1;
    int64_t sA = 0, sB = 0, sC = 0, sBias = 0, sSave = 0;
    // Row strides (elements) of A and B when they are not the packed ones
    // (0: K for a K-contiguous operand, M or N for an M/N-contiguous one); a
    // product over a K range of wider operands.  Tile kernel only.
    int64_t lda = 0, ldb = 0;
};

}  // namespace tpmlp
