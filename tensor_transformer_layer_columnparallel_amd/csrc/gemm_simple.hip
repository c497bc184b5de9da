// General MFMA GEMM for every operand layout, both element types and small or
// ragged shapes: C[M,N] = epi( op(A)[M,K] * op(B)[K,N] ).
//
// 256 threads (4 waves, 2 x 2), a BM x BN output tile per workgroup, BK = 32.
// Operands go global -> VGPR -> LDS.  In LDS both operands are stored with K
// contiguous per row ("k-rows"), so an MFMA fragment is one 16-byte read per
// lane.  An operand stored with M (or N) contiguous in HBM is transposed on
// the way into LDS.  The next K-slab is fetched into registers while the
// current one is multiplied (two LDS stages, one barrier per slab).
//
// bf16 uses v_mfma_f32_16x16x32_bf16, fp32 uses v_mfma_f32_16x16x4_f32; both
// accumulate in fp32.  Lane l of a 16x16 result holds column l % 16 and rows
// 4 * (l / 16) + {0..3}.
#include "common.h"
#include "epilogue.h"
#include "kernels.h"

namespace tpmlp {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = 32;

template <typename T> struct Frag;
template <> struct Frag<bf16> {
    static constexpr int kVec = 8;      // elements per 16-byte vector
    static constexpr int kSteps = 1;    // MFMA k-steps per BK slab (k = 32)
};
template <> struct Frag<float> {
    static constexpr int kVec = 4;
    static constexpr int kSteps = 8;    // k = 4 per MFMA
};

template <typename T>
struct alignas(16) Vec16 {
    T v[16 / sizeof(T)];
};

// Loads one BK slab of an operand into registers.  `rows` is the extent of
// the non-K dimension (M for A, N for B).  K-major: [rows][K] with K
// contiguous; MN-major: [K][rows] with rows contiguous.
template <typename T, bool KMAJ, int BR>
struct SlabLoader {
    static constexpr int kVec = Frag<T>::kVec;
    static constexpr int kChunks = BR * kBK / kVec;
    static constexpr int kPerThread = kChunks / kThreads;
    static_assert(kChunks % kThreads == 0, "tile too small for 256 threads");

    Vec16<T> reg[kPerThread];

    __device__ __forceinline__ void load(const T* __restrict__ g, int64_t rows, int64_t K,
                                         int64_t r0, int64_t k0, int tid)
    {
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            const int c = tid + j * kThreads;
            int64_t r, k;
            if (KMAJ) {
                r = r0 + c / (kBK / kVec);
                k = k0 + (c % (kBK / kVec)) * kVec;
            } else {
                k = k0 + c / (BR / kVec);
                r = r0 + (c % (BR / kVec)) * kVec;
            }
            const bool ok = (r < rows) && (k < K);
            if (ok) {
                const int64_t off = KMAJ ? (r * K + k) : (k * rows + r);
                reg[j] = *reinterpret_cast<const Vec16<T>*>(g + off);
            } else {
#pragma unroll
                for (int e = 0; e < kVec; ++e) reg[j].v[e] = T(0.0f);
            }
        }
    }

    // Writes the registers into an LDS stage laid out [BR][LDK] (k-rows).
    template <int LDK>
    __device__ __forceinline__ void store(T* s, int tid) const
    {
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            const int c = tid + j * kThreads;
            if (KMAJ) {
                const int r = c / (kBK / kVec);
                const int k = (c % (kBK / kVec)) * kVec;
                *reinterpret_cast<Vec16<T>*>(s + r * LDK + k) = reg[j];
            } else {
                const int k = c / (BR / kVec);
                const int r = (c % (BR / kVec)) * kVec;
#pragma unroll
                for (int e = 0; e < kVec; ++e) s[(r + e) * LDK + k] = reg[j].v[e];
            }
        }
    }
};

template <typename T, bool A_KMAJ, bool B_KMAJ, Epi EPI, typename OutT, int BM, int BN>
__global__ __launch_bounds__(kThreads) void gemm_simple_kernel(GemmArgs p)
{
    constexpr int kVec = Frag<T>::kVec;
    constexpr int LDK = kBK + kVec;   // one 16-byte pad per k-row
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int FM = WM / 16, FN = WN / 16;

    __shared__ __attribute__((aligned(16))) T sA[2][BM * LDK];
    __shared__ __attribute__((aligned(16))) T sB[2][BN * LDK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int64_t n0 = (int64_t)blockIdx.x * BN;
    if (p.batch > 1) {
        // product blockIdx.z of a batch: its operands at the batch strides
        const int64_t b = blockIdx.z;
        p.A = static_cast<const T*>(p.A) + b * p.sA;
        p.B = static_cast<const T*>(p.B) + b * p.sB;
        p.C = static_cast<OutT*>(p.C) + b * p.sC;
        if (p.bias) p.bias = static_cast<const T*>(p.bias) + b * p.sBias;
        if (p.save) p.save = static_cast<T*>(p.save) + b * p.sSave;
    }
    const T* __restrict__ A = static_cast<const T*>(p.A);
    const T* __restrict__ B = static_cast<const T*>(p.B);

    SlabLoader<T, A_KMAJ, BM> la;
    SlabLoader<T, B_KMAJ, BN> lb;

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = (int)((p.K + kBK - 1) / kBK);
    if (nk > 0) {
        la.load(A, p.M, p.K, m0, 0, tid);
        lb.load(B, p.N, p.K, n0, 0, tid);
        la.template store<LDK>(sA[0], tid);
        lb.template store<LDK>(sB[0], tid);
        __syncthreads();
    }

    for (int kt = 0; kt < nk; ++kt) {
        const int st = kt & 1;
        const bool more = kt + 1 < nk;
        if (more) {
            la.load(A, p.M, p.K, m0, (int64_t)(kt + 1) * kBK, tid);
            lb.load(B, p.N, p.K, n0, (int64_t)(kt + 1) * kBK, tid);
        }
        const T* a_s = sA[st] + (wm * WM) * LDK;
        const T* b_s = sB[st] + (wn * WN) * LDK;
        if constexpr (sizeof(T) == 2) {
            bf16x8 af[FM], bfr[FN];
            const int row = lane & 15, kof = (lane >> 4) * 8;
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = *reinterpret_cast<const bf16x8*>(a_s + (i * 16 + row) * LDK + kof);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8*>(b_s + (j * 16 + row) * LDK + kof);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        } else {
            const int row = lane & 15, kof = lane >> 4;
#pragma unroll
            for (int s = 0; s < Frag<T>::kSteps; ++s) {
                float af[FM], bfr[FN];
#pragma unroll
                for (int i = 0; i < FM; ++i) af[i] = a_s[(i * 16 + row) * LDK + s * 4 + kof];
#pragma unroll
                for (int j = 0; j < FN; ++j) bfr[j] = b_s[(j * 16 + row) * LDK + s * 4 + kof];
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i], bfr[j], acc[i][j], 0, 0, 0);
            }
        }
        if (more) {
            la.template store<LDK>(sA[st ^ 1], tid);
            lb.template store<LDK>(sB[st ^ 1], tid);
        }
        __syncthreads();
    }

    // Epilogue: lane holds column (lane % 16), rows 4 * (lane / 16) + e.
    OutT* __restrict__ C = static_cast<OutT*>(p.C);
    const T* __restrict__ bias = static_cast<const T*>(p.bias);
    const T* __restrict__ aux = static_cast<const T*>(p.aux);
    T* __restrict__ save = static_cast<T*>(p.save);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int64_t col = n0 + wn * WN + j * 16 + (lane & 15);
        if (col >= p.N) continue;
        float bcol = 0.f;
        if constexpr (EPI == Epi::Bias || EPI == Epi::BiasGelu) {
            if (bias) bcol = to_f32(bias[col]);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t row = m0 + wm * WM + i * 16 + (lane >> 4) * 4 + e;
                if (row >= p.M) continue;
                const int64_t off = EPI == Epi::StoreT ? col * p.M + row : row * p.N + col;
                float v = acc[i][j][e];
                if constexpr (EPI == Epi::Bias) {
                    v += bcol;
                } else if constexpr (EPI == Epi::BiasGelu) {
                    v += bcol;
                    if (save) save[off] = from_f32<T>(v);
                    v = gelu_tanh(v);
                } else if constexpr (EPI == Epi::DGelu) {
                    v *= gelu_tanh_grad(to_f32(aux[off]));
                }
                C[off] = from_f32<OutT>(v);
            }
        }
    }
}

template <typename T, bool A_KMAJ, bool B_KMAJ, Epi EPI, typename OutT, int BM, int BN>
hipError_t launch_tile(const GemmArgs& p, hipStream_t stream)
{
    if ((p.M + BM - 1) / BM > 65535) return hipErrorInvalidValue;   // grid y
    dim3 grid((unsigned)((p.N + BN - 1) / BN), (unsigned)((p.M + BM - 1) / BM),
              (unsigned)p.batch);
    hipLaunchKernelGGL((gemm_simple_kernel<T, A_KMAJ, B_KMAJ, EPI, OutT, BM, BN>), grid,
                       dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

// 128 x 128 tiles, or smaller ones (64 x 64; 32 x 32 for fp32, whose slab
// of 32 rows fills the 256 threads' loads) when the larger tiles would leave
// most of the 256 CUs idle: a product of a few rows (the tiny fp32 layer's
// 32 tokens) otherwise runs its whole K loop on a tile that is mostly
// padding, on a handful of CUs.  Every output sums k in the same order
// whatever the tile, so the results are the same bits.
template <typename T, bool A_KMAJ, bool B_KMAJ, Epi EPI, typename OutT>
hipError_t launch(const GemmArgs& p, hipStream_t stream)
{
    auto tiles = [&](int64_t b) { return ((p.M + b - 1) / b) * ((p.N + b - 1) / b) * p.batch; };
    constexpr int64_t kFew = 128;   // half the CUs
    if (tiles(128) >= kFew) return launch_tile<T, A_KMAJ, B_KMAJ, EPI, OutT, 128, 128>(p, stream);
    if constexpr (sizeof(T) == 2) {
        return launch_tile<T, A_KMAJ, B_KMAJ, EPI, OutT, 64, 64>(p, stream);
    } else {
        if (tiles(64) >= kFew) return launch_tile<T, A_KMAJ, B_KMAJ, EPI, OutT, 64, 64>(p, stream);
        return launch_tile<T, A_KMAJ, B_KMAJ, EPI, OutT, 32, 32>(p, stream);
    }
}

}  // namespace

hipError_t gemm_simple(const GemmArgs& p, Elt elt, Layout layout, Epi epi, Elt out,
                       hipStream_t stream)
{
    if (p.lda || p.ldb) return hipErrorInvalidValue;   // packed operands only
    // A batch of products runs as one launch, grid z = product (in launches of
    // at most 65535 products, the grid's z limit).
    if (p.batch < 1) return hipErrorInvalidValue;
    if (p.batch > 1 && epi != Epi::Store && epi != Epi::Bias && epi != Epi::BiasGelu)
        return hipErrorInvalidValue;
    constexpr int64_t kMaxZ = 65535;
    if (p.batch > kMaxZ) {
        const int64_t es = elt == Elt::F32 ? 4 : 2, os = out == Elt::F32 ? 4 : 2;
        for (int64_t b0 = 0; b0 < p.batch; b0 += kMaxZ) {
            GemmArgs q = p;
            q.batch = p.batch - b0 < kMaxZ ? p.batch - b0 : kMaxZ;
            q.A = static_cast<const char*>(p.A) + b0 * p.sA * es;
            q.B = static_cast<const char*>(p.B) + b0 * p.sB * es;
            q.C = static_cast<char*>(p.C) + b0 * p.sC * os;
            if (p.bias) q.bias = static_cast<const char*>(p.bias) + b0 * p.sBias * es;
            if (p.save) q.save = static_cast<char*>(p.save) + b0 * p.sSave * es;
            const hipError_t e = gemm_simple(q, elt, layout, epi, out, stream);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
#define TP_CASE(T, AK, BK_, E, O)                                                    \
    return launch<T, AK, BK_, E, O>(p, stream)
    if (elt == Elt::F32) {
        if (out != Elt::F32) return hipErrorInvalidValue;
        switch (layout) {
        case Layout::NN:
            if (epi == Epi::BiasGelu) TP_CASE(float, true, false, Epi::BiasGelu, float);
            if (epi == Epi::Bias) TP_CASE(float, true, false, Epi::Bias, float);
            if (epi == Epi::StoreT) TP_CASE(float, true, false, Epi::StoreT, float);
            TP_CASE(float, true, false, Epi::Store, float);
        case Layout::NT:
            if (epi == Epi::DGelu) TP_CASE(float, true, true, Epi::DGelu, float);
            TP_CASE(float, true, true, Epi::Store, float);
        case Layout::TN:
            TP_CASE(float, false, false, Epi::Store, float);
        }
    } else {
        switch (layout) {
        case Layout::NN:
            if (epi == Epi::BiasGelu) {
                if (out == Elt::BF16) TP_CASE(bf16, true, false, Epi::BiasGelu, bf16);
                TP_CASE(bf16, true, false, Epi::BiasGelu, float);
            }
            if (epi == Epi::Bias) {
                if (out == Elt::BF16) TP_CASE(bf16, true, false, Epi::Bias, bf16);
                TP_CASE(bf16, true, false, Epi::Bias, float);
            }
            if (epi == Epi::StoreT) {
                if (out != Elt::F32) return hipErrorInvalidValue;
                TP_CASE(bf16, true, false, Epi::StoreT, float);
            }
            if (out == Elt::BF16) TP_CASE(bf16, true, false, Epi::Store, bf16);
            TP_CASE(bf16, true, false, Epi::Store, float);
        case Layout::NT:
            if (epi == Epi::DGelu) {
                if (out == Elt::BF16) TP_CASE(bf16, true, true, Epi::DGelu, bf16);
                TP_CASE(bf16, true, true, Epi::DGelu, float);
            }
            if (out == Elt::BF16) TP_CASE(bf16, true, true, Epi::Store, bf16);
            TP_CASE(bf16, true, true, Epi::Store, float);
        case Layout::TN:
            TP_CASE(bf16, false, false, Epi::Store, float);
        }
    }
#undef TP_CASE
    return hipErrorInvalidValue;
}

}  // namespace tpmlp
