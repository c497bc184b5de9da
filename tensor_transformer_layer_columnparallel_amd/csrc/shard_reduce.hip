// HBM-streaming kernels: the on-device stand-ins for the collectives between
// ranks (sum of row-parallel partials, concatenation of column shards) and
// the bias gradient (a column sum).  None of them uses LDS tiling beyond a
// final fixed-order combine, and none uses atomics, so every result is
// bitwise reproducible from run to run.
#include "common.h"
#include "kernels.h"

namespace tpmlp {
namespace {

constexpr int kThreads = 256;

// 8 consecutive elements, loaded or stored as 16-byte vectors.
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
    *reinterpret_cast<f32x4*>(p) = f32x4{o.v[0], o.v[1], o.v[2], o.v[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{o.v[4], o.v[5], o.v[6], o.v[7]};
}
__device__ __forceinline__ void store8(bf16* p, const Oct& o)
{
    bf16x8 a;
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = (bf16)o.v[e];
    *reinterpret_cast<bf16x8*>(p) = a;
}

// Streaming forms of the loads and stores above: every byte of the partials
// is read once and every output written once, so they are marked
// non-temporal (8% faster on the 1.2 GB sum of eight [4096, 8192] fp32
// partials than ordinary loads and stores).
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
__device__ __forceinline__ void store8_nt(float* p, const Oct& o)
{
    __builtin_nontemporal_store(f32x4{o.v[0], o.v[1], o.v[2], o.v[3]},
                                reinterpret_cast<f32x4*>(p));
    __builtin_nontemporal_store(f32x4{o.v[4], o.v[5], o.v[6], o.v[7]},
                                reinterpret_cast<f32x4*>(p + 4));
}
__device__ __forceinline__ void store8_nt(bf16* p, const Oct& o)
{
    bf16x8 a;
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = (bf16)o.v[e];
    __builtin_nontemporal_store(__builtin_bit_cast(i32x4, a), reinterpret_cast<i32x4*>(p));
}

// out[e] = parts[0][e] + ... + parts[t-1][e], parts[r] starting `stride`
// elements after parts[r-1].  TT > 0: t == TT known at compile time, so all t
// loads of a vector are issued before the adds.
// A one-part sum is a copy with the type conversion (the token
// concatenation): each thread moves kCopyOcts octets, their loads issued
// before the stores.  Two octets per thread: [8][256][12288] -> [2048][12288]
// fp32 51.7 -> 39.3 us (3.9 -> 5.1 TB/s), bf16 18.05 -> 17.94 us; four were
// slower for both.
constexpr int kCopyOcts = 2;

template <typename In, typename Out, int TT>
__global__ __launch_bounds__(kThreads) void shard_sum_kernel(const In* __restrict__ parts,
                                                             Out* __restrict__ out,
                                                             int64_t nvec, int64_t stride, int t)
{
    if constexpr (TT == 1) {
        const int64_t span = (int64_t)kThreads * kCopyOcts;
        for (int64_t v0 = (int64_t)blockIdx.x * span + threadIdx.x; v0 < nvec;
             v0 += (int64_t)gridDim.x * span) {
            Oct x[kCopyOcts];
#pragma unroll
            for (int i = 0; i < kCopyOcts; ++i) {
                const int64_t v = v0 + (int64_t)i * kThreads;
                if (v < nvec) x[i] = load8_nt(parts + v * 8);
            }
#pragma unroll
            for (int i = 0; i < kCopyOcts; ++i) {
                const int64_t v = v0 + (int64_t)i * kThreads;
                if (v < nvec) store8_nt(out + v * 8, x[i]);
            }
        }
        return;
    }
    const int64_t step = (int64_t)gridDim.x * kThreads;
    for (int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x; v < nvec; v += step) {
        const int64_t e0 = v * 8;
        Oct s;
        if constexpr (TT > 0) {
            Oct x[TT];
#pragma unroll
            for (int r = 0; r < TT; ++r) x[r] = load8_nt(parts + (int64_t)r * stride + e0);
            s = x[0];
#pragma unroll
            for (int r = 1; r < TT; ++r)
#pragma unroll
                for (int e = 0; e < 8; ++e) s.v[e] += x[r].v[e];
        } else {
            s = load8_nt(parts + e0);
            for (int r = 1; r < t; ++r) {
                const Oct x = load8_nt(parts + (int64_t)r * stride + e0);
#pragma unroll
                for (int e = 0; e < 8; ++e) s.v[e] += x.v[e];
            }
        }
        store8_nt(out + e0, s);
    }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void shard_concat_kernel(const T* __restrict__ parts,
                                                                T* __restrict__ out, int64_t rows,
                                                                int64_t cols, int t)
{
    const int64_t pairs = rows * t;
    const int64_t c8 = cols / 8;
    for (int64_t q = blockIdx.x; q < pairs; q += gridDim.x) {
        const int64_t m = q / t;
        const int r = (int)(q - m * t);
        const T* src = parts + ((int64_t)r * rows + m) * cols;
        T* dst = out + m * (cols * t) + (int64_t)r * cols;
        // 8 elements per step: one 16-byte vector for bf16, two for fp32.
        for (int64_t c = threadIdx.x; c < c8; c += kThreads) {
#pragma unroll
            for (int h = 0; h < (int)sizeof(T) / 2; ++h)
                *reinterpret_cast<i32x4*>(dst + c * 8 + h * 4) =
                    *reinterpret_cast<const i32x4*>(src + c * 8 + h * 4);
        }
    }
}

// Column sums: 8 consecutive columns per thread, kRowGroups threads per
// column octet stepping through rows, combined in LDS in fixed order.
constexpr int kColOcts = 8;                       // 64 columns per block
constexpr int kRowGroups = kThreads / kColOcts;   // 32

template <typename T>
__global__ __launch_bounds__(kThreads) void column_sum_kernel(const T* __restrict__ in,
                                                              float* __restrict__ out,
                                                              int64_t rows, int64_t cols)
{
    __shared__ float part[kRowGroups][kColOcts * 8];
    const int oct = threadIdx.x % kColOcts;
    const int rg = threadIdx.x / kColOcts;
    const int64_t c0 = (int64_t)blockIdx.x * kColOcts * 8 + oct * 8;
    Oct s{{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}};
    if (c0 < cols) {
        for (int64_t m = rg; m < rows; m += kRowGroups) {
            const Oct x = load8(in + m * cols + c0);
#pragma unroll
            for (int e = 0; e < 8; ++e) s.v[e] += x.v[e];
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[rg][oct * 8 + e] = s.v[e];
    __syncthreads();
    if (threadIdx.x < kColOcts * 8) {
        const int64_t c = (int64_t)blockIdx.x * kColOcts * 8 + threadIdx.x;
        float acc = 0.f;
        for (int g = 0; g < kRowGroups; ++g) acc += part[g][threadIdx.x];
        if (c < cols) out[c] = acc;
    }
}

// Two-level column sums for tall inputs: row blocks of kSumRows rows give
// partial sums (512 columns x 64 rows per workgroup, so that every CU gets
// work), then one thread per column adds the partials in row-block order.
constexpr int kSumRows = 64;
constexpr int kSumOcts = 64;                              // 512 columns per workgroup
constexpr int kSumSub = kThreads / kSumOcts;              // 4 row subgroups

template <typename T>
__global__ __launch_bounds__(kThreads) void column_part_kernel(const T* __restrict__ in,
                                                               float* __restrict__ part,
                                                               int64_t rows, int64_t cols,
                                                               int64_t col_blocks)
{
    __shared__ float red[kSumSub][kSumOcts * 8];
    const int64_t rb = blockIdx.x / col_blocks, cb = blockIdx.x % col_blocks;
    const int oct = threadIdx.x % kSumOcts, sub = threadIdx.x / kSumOcts;
    const int64_t c0 = cb * kSumOcts * 8 + oct * 8;
    Oct s{{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}};
    if (c0 < cols) {
        const int64_t m_end = (rb + 1) * kSumRows < rows ? (rb + 1) * kSumRows : rows;
        int64_t m = rb * kSumRows + sub;
        // Four rows' loads in flight at a time; the adds stay in row order.
        for (; m + 3 * kSumSub < m_end; m += 4 * kSumSub) {
            Oct x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) x[u] = load8(in + (m + u * kSumSub) * cols + c0);
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int e = 0; e < 8; ++e) s.v[e] += x[u].v[e];
        }
        for (; m < m_end; m += kSumSub) {
            const Oct x = load8(in + m * cols + c0);
#pragma unroll
            for (int e = 0; e < 8; ++e) s.v[e] += x.v[e];
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[sub][oct * 8 + e] = s.v[e];
    __syncthreads();
    for (int c = threadIdx.x; c < kSumOcts * 8; c += kThreads) {
        const int64_t col = cb * kSumOcts * 8 + c;
        if (col >= cols) break;
        float acc = 0.f;
#pragma unroll
        for (int g = 0; g < kSumSub; ++g) acc += red[g][c];
        part[rb * cols + col] = acc;
    }
}

__global__ __launch_bounds__(kThreads) void column_final_kernel(const float* __restrict__ part,
                                                                float* __restrict__ out,
                                                                int64_t nrb, int64_t cols)
{
    const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (c < cols) column_finish_one(part, out, nrb, cols, c);
}

unsigned stream_grid(int64_t work_items)
{
    const int64_t cap = 256 * 16;   // 16 workgroups per CU, grid-stride beyond
    const int64_t g = (work_items + kThreads - 1) / kThreads;
    return (unsigned)(g < 1 ? 1 : (g > cap ? cap : g));
}

template <typename In, typename Out>
hipError_t sum_launch(const void* parts, void* out, int64_t count, int64_t stride, int t,
                      hipStream_t s)
{
    const int64_t nvec = count / 8;
    // One octet per thread, kCopyOcts for a one-part copy (grid-stride only
    // past 2^20 workgroups): 4% faster on the eight-partial sum than 16
    // workgroups per CU striding.
    const int64_t per_block = t == 1 ? (int64_t)kThreads * kCopyOcts : kThreads;
    const int64_t g = (nvec + per_block - 1) / per_block;
    const dim3 grid((unsigned)(g > (1 << 20) ? (1 << 20) : g)), block(kThreads);
    const In* p = static_cast<const In*>(parts);
    Out* o = static_cast<Out*>(out);
    switch (t) {
    case 1: hipLaunchKernelGGL((shard_sum_kernel<In, Out, 1>), grid, block, 0, s, p, o, nvec, stride, t); break;
    case 2: hipLaunchKernelGGL((shard_sum_kernel<In, Out, 2>), grid, block, 0, s, p, o, nvec, stride, t); break;
    case 4: hipLaunchKernelGGL((shard_sum_kernel<In, Out, 4>), grid, block, 0, s, p, o, nvec, stride, t); break;
    case 8: hipLaunchKernelGGL((shard_sum_kernel<In, Out, 8>), grid, block, 0, s, p, o, nvec, stride, t); break;
    default: hipLaunchKernelGGL((shard_sum_kernel<In, Out, 0>), grid, block, 0, s, p, o, nvec, stride, t); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t shard_sum(const void* parts, void* out, int64_t count, int64_t stride, int t, Elt in,
                     Elt out_elt, hipStream_t stream)
{
    if (count <= 0) return hipSuccess;
    if (in == Elt::F32 && out_elt == Elt::F32) return sum_launch<float, float>(parts, out, count, stride, t, stream);
    if (in == Elt::F32 && out_elt == Elt::BF16) return sum_launch<float, bf16>(parts, out, count, stride, t, stream);
    if (in == Elt::BF16 && out_elt == Elt::F32) return sum_launch<bf16, float>(parts, out, count, stride, t, stream);
    return sum_launch<bf16, bf16>(parts, out, count, stride, t, stream);
}

hipError_t shard_concat(const void* parts, void* out, int64_t rows, int64_t cols, int t,
                        Elt elt, hipStream_t stream)
{
    if (rows <= 0) return hipSuccess;
    const int64_t pairs = rows * t;
    const unsigned grid = (unsigned)(pairs < 256 * 16 ? pairs : 256 * 16);
    if (elt == Elt::F32)
        hipLaunchKernelGGL((shard_concat_kernel<float>), dim3(grid), dim3(kThreads), 0, stream,
                           static_cast<const float*>(parts), static_cast<float*>(out), rows, cols, t);
    else
        hipLaunchKernelGGL((shard_concat_kernel<bf16>), dim3(grid), dim3(kThreads), 0, stream,
                           static_cast<const bf16*>(parts), static_cast<bf16*>(out), rows, cols, t);
    return hipGetLastError();
}

hipError_t column_sum(const void* in, float* out, int64_t rows, int64_t cols, Elt elt,
                      void* scratch, int64_t scratch_bytes, hipStream_t stream)
{
    const int64_t nrb = (rows + kSumRows - 1) / kSumRows;
    const int64_t col_blocks = (cols + kSumOcts * 8 - 1) / (kSumOcts * 8);
    if (scratch && nrb > 1 && nrb * cols * 4 <= scratch_bytes && nrb * col_blocks <= INT32_MAX) {
        float* part = static_cast<float*>(scratch);
        const dim3 grid((unsigned)(nrb * col_blocks));
        if (elt == Elt::F32)
            hipLaunchKernelGGL((column_part_kernel<float>), grid, dim3(kThreads), 0, stream,
                               static_cast<const float*>(in), part, rows, cols, col_blocks);
        else
            hipLaunchKernelGGL((column_part_kernel<bf16>), grid, dim3(kThreads), 0, stream,
                               static_cast<const bf16*>(in), part, rows, cols, col_blocks);
        hipLaunchKernelGGL(column_final_kernel, dim3((unsigned)((cols + kThreads - 1) / kThreads)),
                           dim3(kThreads), 0, stream, part, out, nrb, cols);
        return hipGetLastError();
    }
    const unsigned grid = (unsigned)((cols + kColOcts * 8 - 1) / (kColOcts * 8));
    if (elt == Elt::F32)
        hipLaunchKernelGGL((column_sum_kernel<float>), dim3(grid), dim3(kThreads), 0, stream,
                           static_cast<const float*>(in), out, rows, cols);
    else
        hipLaunchKernelGGL((column_sum_kernel<bf16>), dim3(grid), dim3(kThreads), 0, stream,
                           static_cast<const bf16*>(in), out, rows, cols);
    return hipGetLastError();
}

hipError_t column_finish(const float* part, float* out, int64_t nparts, int64_t cols,
                         hipStream_t stream)
{
    if (cols <= 0) return hipSuccess;
    hipLaunchKernelGGL(column_final_kernel, dim3((unsigned)((cols + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, stream, part, out, nparts, cols);
    return hipGetLastError();
}

}  // namespace tpmlp
