// Layer normalisation of whole rows, the normalisation a sequence-parallel
// rank applies to its token shard (alone, or fused with the ReduceScatter that
// produces the shard, its rows summed from the t partials as they are
// loaded): one workgroup per row, fp32 statistics
// (mean, then the biased variance around it), fixed reduction order (so the
// result is bitwise reproducible), 16-byte vector loads and stores, the
// results written with non-temporal stores (the [256, 12288] fp32 -> bf16
// shard 17% faster than with plain stores: 7.3 -> 6.1 us).  Rows of
// up to kThreads * kMaxOcts * 8 columns are held in registers (one read of
// HBM); longer rows are read three times, the later passes from L2.
#include "common.h"
#include "kernels.h"

namespace tpmlp {
namespace {

// 1024 threads (16 waves) per row: more loads issued at once per CU than
// with 512 (3% faster on a [256, 12288] fp32 shard, where every row is one
// CU's only work; 256 threads were 29% slower).
constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxOcts = 4;   // register-resident row: up to 32768 columns

struct Oct {
    float v[8];
};

__device__ __forceinline__ Oct load8(const float* p)
{
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    return Oct{{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]}};
}
__device__ __forceinline__ Oct load8(const bf16* p)
{
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(p);
    Oct o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o.v[e] = (float)a[e];
    return o;
}
__device__ __forceinline__ void store8(float* p, const Oct& o)
{
    __builtin_nontemporal_store(f32x4{o.v[0], o.v[1], o.v[2], o.v[3]}, reinterpret_cast<f32x4*>(p));
    __builtin_nontemporal_store(f32x4{o.v[4], o.v[5], o.v[6], o.v[7]}, reinterpret_cast<f32x4*>(p + 4));
}
__device__ __forceinline__ void store8(bf16* p, const Oct& o)
{
    bf16x8 a;
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = (bf16)o.v[e];
    __builtin_nontemporal_store(__builtin_bit_cast(i32x4, a), reinterpret_cast<i32x4*>(p));
}

// Non-temporal loads for the summed rows: every byte of the partials is read
// once.
__device__ __forceinline__ Oct load8_nt(const float* p)
{
    const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
    return Oct{{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]}};
}
__device__ __forceinline__ Oct load8_nt(const bf16* p)
{
    const i32x4 w = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(p));
    const bf16x8 a = __builtin_bit_cast(bf16x8, w);
    Oct o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o.v[e] = (float)a[e];
    return o;
}

// Where a row's values come from.  RowLoad: row m of x.  SumLoad: row m of a
// rank's token block of the sum of t partials, added in fp32 in rank order
// 0..t-1 (TT = t when it is known at compile time, so that all t loads of
// an octet are issued before the adds; 0 otherwise) -- the values
// tp_shard_reduce_scatter writes with an fp32 output.
template <typename In>
struct RowLoad {
    const In* x;
    int64_t cols;
    __device__ __forceinline__ Oct operator()(int64_t m, int64_t c8) const
    {
        return load8(x + m * cols + c8 * 8);
    }
};
template <typename In, int TT>
struct SumLoad {
    const In* parts;   // parts[0] + rank * rows * cols: the rank's first row
    int64_t cols, stride;
    int t;
    __device__ __forceinline__ Oct operator()(int64_t m, int64_t c8) const
    {
        const In* q = parts + m * cols + c8 * 8;
        Oct s;
        if constexpr (TT > 0) {
            Oct x[TT];
#pragma unroll
            for (int r = 0; r < TT; ++r) x[r] = load8_nt(q + (int64_t)r * stride);
            s = x[0];
#pragma unroll
            for (int r = 1; r < TT; ++r)
#pragma unroll
                for (int e = 0; e < 8; ++e) s.v[e] += x[r].v[e];
        } else {
            s = load8_nt(q);
            for (int r = 1; r < t; ++r) {
                const Oct x = load8_nt(q + (int64_t)r * stride);
#pragma unroll
                for (int e = 0; e < 8; ++e) s.v[e] += x.v[e];
            }
        }
        return s;
    }
};

// Sum over the workgroup: a butterfly inside each wave (every lane ends with
// the same value, in a fixed order), then the wave totals in wave order.
// Each of a row's two sums has its own `red`, so one barrier per sum.
__device__ __forceinline__ float block_sum(float v, float* red)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s += red[w];
    return s;
}

template <typename Load, typename Out>
__global__ __launch_bounds__(kThreads) void layernorm_kernel(Load load,
                                                             const Out* __restrict__ gamma,
                                                             const Out* __restrict__ beta,
                                                             Out* __restrict__ y, int64_t rows,
                                                             int64_t cols, float eps)
{
    __shared__ float red[2][kWaves];
    const int64_t m = blockIdx.x;
    if (m >= rows) return;
    Out* yr = y + m * cols;
    const int64_t c8 = cols / 8;

    float s = 0.f;
    for (int64_t c = threadIdx.x; c < c8; c += kThreads) {
        const Oct o = load(m, c);
#pragma unroll
        for (int e = 0; e < 8; ++e) s += o.v[e];
    }
    const float mean = block_sum(s, red[0]) / (float)cols;

    float q = 0.f;
    for (int64_t c = threadIdx.x; c < c8; c += kThreads) {
        const Oct o = load(m, c);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float d = o.v[e] - mean;
            q += d * d;
        }
    }
    const float var = block_sum(q, red[1]) / (float)cols;
    const float inv = 1.0f / sqrtf(var + eps);

    for (int64_t c = threadIdx.x; c < c8; c += kThreads) {
        Oct o = load(m, c);
        Oct g, b;
        if (gamma) g = load8(gamma + c * 8);
        if (beta) b = load8(beta + c * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = (o.v[e] - mean) * inv;
            if (gamma) v *= g.v[e];
            if (beta) v += b.v[e];
            o.v[e] = v;
        }
        store8(yr + c * 8, o);
    }
}

// Register-resident variant: thread i holds octets i, i + kThreads, ...
template <typename Load, typename Out, int NOCT>
__global__ __launch_bounds__(kThreads) void layernorm_reg_kernel(Load load,
                                                                 const Out* __restrict__ gamma,
                                                                 const Out* __restrict__ beta,
                                                                 Out* __restrict__ y,
                                                                 int64_t rows, int64_t cols,
                                                                 float eps)
{
    __shared__ float red[2][kWaves];
    const int64_t m = blockIdx.x;
    if (m >= rows) return;
    Out* yr = y + m * cols;
    const int c8 = (int)(cols / 8);
    Oct o[NOCT];
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < NOCT; ++j) {
        const int c = threadIdx.x + j * kThreads;
        if (c < c8) {
            o[j] = load(m, c);
#pragma unroll
            for (int e = 0; e < 8; ++e) s += o[j].v[e];
        }
    }
    const float mean = block_sum(s, red[0]) / (float)cols;
    float q = 0.f;
#pragma unroll
    for (int j = 0; j < NOCT; ++j) {
        const int c = threadIdx.x + j * kThreads;
        if (c < c8) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float d = o[j].v[e] - mean;
                q += d * d;
            }
        }
    }
    const float var = block_sum(q, red[1]) / (float)cols;
    const float inv = 1.0f / sqrtf(var + eps);
#pragma unroll
    for (int j = 0; j < NOCT; ++j) {
        const int c = threadIdx.x + j * kThreads;
        if (c < c8) {
            Oct g, b;
            if (gamma) g = load8(gamma + (int64_t)c * 8);
            if (beta) b = load8(beta + (int64_t)c * 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float v = (o[j].v[e] - mean) * inv;
                if (gamma) v *= g.v[e];
                if (beta) v += b.v[e];
                o[j].v[e] = v;
            }
            store8(yr + (int64_t)c * 8, o[j]);
        }
    }
}

template <typename Load, typename Out>
hipError_t launch(const Load& load, const void* gamma, const void* beta, void* y, int64_t rows,
                  int64_t cols, float eps, hipStream_t stream)
{
    const dim3 grid((unsigned)rows), block(kThreads);
    const Out *g = static_cast<const Out*>(gamma), *b = static_cast<const Out*>(beta);
    Out* yo = static_cast<Out*>(y);
    const int64_t c8 = cols / 8;
    if (c8 <= kThreads)
        hipLaunchKernelGGL((layernorm_reg_kernel<Load, Out, 1>), grid, block, 0, stream, load, g, b, yo, rows, cols, eps);
    else if (c8 <= 2 * kThreads)
        hipLaunchKernelGGL((layernorm_reg_kernel<Load, Out, 2>), grid, block, 0, stream, load, g, b, yo, rows, cols, eps);
    else if (c8 <= kMaxOcts * kThreads)
        hipLaunchKernelGGL((layernorm_reg_kernel<Load, Out, kMaxOcts>), grid, block, 0, stream, load, g, b, yo, rows, cols, eps);
    else
        hipLaunchKernelGGL((layernorm_kernel<Load, Out>), grid, block, 0, stream, load, g, b, yo, rows, cols, eps);
    return hipGetLastError();
}

template <typename In, typename Out>
hipError_t launch_rows(const void* x, const void* gamma, const void* beta, void* y, int64_t rows,
                       int64_t cols, float eps, hipStream_t stream)
{
    return launch<RowLoad<In>, Out>(RowLoad<In>{static_cast<const In*>(x), cols}, gamma, beta, y,
                                    rows, cols, eps, stream);
}

template <typename In, typename Out>
hipError_t launch_sum(const void* parts, int64_t stride, int t, const void* gamma,
                      const void* beta, void* y, int64_t rows, int64_t cols, float eps,
                      hipStream_t stream)
{
    const In* p = static_cast<const In*>(parts);
    switch (t) {
    case 1: return launch<SumLoad<In, 1>, Out>(SumLoad<In, 1>{p, cols, stride, t}, gamma, beta, y, rows, cols, eps, stream);
    case 2: return launch<SumLoad<In, 2>, Out>(SumLoad<In, 2>{p, cols, stride, t}, gamma, beta, y, rows, cols, eps, stream);
    case 4: return launch<SumLoad<In, 4>, Out>(SumLoad<In, 4>{p, cols, stride, t}, gamma, beta, y, rows, cols, eps, stream);
    case 8: return launch<SumLoad<In, 8>, Out>(SumLoad<In, 8>{p, cols, stride, t}, gamma, beta, y, rows, cols, eps, stream);
    default: return launch<SumLoad<In, 0>, Out>(SumLoad<In, 0>{p, cols, stride, t}, gamma, beta, y, rows, cols, eps, stream);
    }
}

}  // namespace

hipError_t layernorm(const void* x, const void* gamma, const void* beta, void* y, int64_t rows,
                     int64_t cols, float eps, Elt in, Elt out, hipStream_t stream)
{
    if (rows == 0) return hipSuccess;
    if (rows > INT32_MAX) return hipErrorInvalidValue;
    if (in == Elt::F32 && out == Elt::F32) return launch_rows<float, float>(x, gamma, beta, y, rows, cols, eps, stream);
    if (in == Elt::F32 && out == Elt::BF16) return launch_rows<float, bf16>(x, gamma, beta, y, rows, cols, eps, stream);
    if (in == Elt::BF16 && out == Elt::F32) return launch_rows<bf16, float>(x, gamma, beta, y, rows, cols, eps, stream);
    return launch_rows<bf16, bf16>(x, gamma, beta, y, rows, cols, eps, stream);
}

hipError_t sum_layernorm(const void* parts, int64_t stride, int t, const void* gamma,
                         const void* beta, void* y, int64_t rows, int64_t cols, float eps, Elt in,
                         Elt out, hipStream_t stream)
{
    if (rows == 0) return hipSuccess;
    if (rows > INT32_MAX || t < 1) return hipErrorInvalidValue;
    if (in == Elt::F32 && out == Elt::F32) return launch_sum<float, float>(parts, stride, t, gamma, beta, y, rows, cols, eps, stream);
    if (in == Elt::F32 && out == Elt::BF16) return launch_sum<float, bf16>(parts, stride, t, gamma, beta, y, rows, cols, eps, stream);
    if (in == Elt::BF16 && out == Elt::F32) return launch_sum<bf16, float>(parts, stride, t, gamma, beta, y, rows, cols, eps, stream);
    return launch_sum<bf16, bf16>(parts, stride, t, gamma, beta, y, rows, cols, eps, stream);
}

}  // namespace tpmlp
