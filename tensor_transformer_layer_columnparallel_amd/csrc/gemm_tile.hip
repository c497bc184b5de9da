// Large-tile bf16 MFMA GEMM for gfx950: C[M,N] = epi( op(A)[M,K] * op(B)[K,N] ).
//
// Workgroup: 512 threads = 8 waves (two per SIMD) in a 4 x 2 grid, a
// 256 x BN output tile per workgroup (BN = 256 or 192), 64 x BN/2 per wave
// (4 x BN/32 MFMA 16x16x32 bf16 tiles, fp32 accumulators).  K advances in
// slabs of 64.  Two waves per SIMD let one wave's LDS and barrier waits
// overlap the other's MFMAs.
// BN = 192 exists for wave quantisation: the six products of the GPT-3-shaped
// shard (M = 2048 with N = 6144 or 12288, and the 6144 x 12288 weight
// gradients) all split into whole multiples of 256 tiles of 256 x 192.
//
// HBM -> LDS: buffer_load_dwordx4 ... lds (each lane's 16 bytes land directly
// in LDS, no VGPR staging).  Elements outside the operand (ragged M, N or K
// tails) are given a per-lane offset beyond the buffer descriptor's extent,
// which returns zeros; every other address stays inside the operand.  Two LDS stages: slab k+1 streams in while slab k is multiplied.
// (All LDS reads of a stage are issued before the DMA into the other stage:
// the compiler cannot tell the two stages apart and waits for the DMA
// before any LDS read that follows it in program order.)
//
// LDS layouts (16-byte chunks permuted per row so that fragment reads are
// free of bank conflicts):
//   K-major operand  [rows][64 k]     read with ds_read_b128 (8 k per lane)
//   MN-major operand [64 k][rows]     read with ds_read_b64_tr_b16: within a
//     16-lane group, lane i receives element (i % 4) of the 8-byte pieces
//     loaded by lanes 4e + i/4, e = 0..3.  Pointing lane 4e + g at
//     row k0 + e, columns 4g..4g+3 gives every lane four consecutive k of
//     one column: half of an MFMA operand; two reads make the 8.
//
// The MFMA is issued with the B fragment in the first operand slot and the A
// fragment in the second, so a lane's four results are four consecutive
// columns of one output row (16-byte fp32 / 8-byte bf16 stores).
//
// Workgroups are remapped so that consecutive output tiles, which share
// operand panels, run on the same XCD (hardware dispatches workgroup w to
// XCD w % 8) and hit that XCD's L2.
#include "common.h"
#include "epilogue.h"
#include "kernels.h"

namespace tpmlp {
namespace {

constexpr int kBM = 256;
constexpr int kBK = 64;
constexpr int kXcds = 8;
#ifndef TPMLP_TILE_WAVES_M
#define TPMLP_TILE_WAVES_M 4
#endif
#ifndef TPMLP_TILE_WAVES_N
#define TPMLP_TILE_WAVES_N 2
#endif
constexpr int kWavesM = TPMLP_TILE_WAVES_M;   // wave grid of a workgroup
constexpr int kWavesN = TPMLP_TILE_WAVES_N;
constexpr int kWaves = kWavesM * kWavesN;
constexpr int kThreads = 64 * kWaves;

// Third descriptor word of a raw buffer resource on gfx9-family GPUs.
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             kRsrcWord3);
}

__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rsrc, bf16* lds_base,
                                           uint32_t voffset, uint32_t soffset)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (TP_LDS void*)lds_base, 16, voffset, soffset,
                                             0, 0);
}

// K-major slab [R rows][64 k]: 8 chunks per row, XOR-permuted by row so that
// the 16 rows read by one 16-lane group hit distinct banks (whether the LDS
// serves 8 or 16 lanes of a 16-byte read per cycle).
__device__ __forceinline__ int swz_kmaj(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// MN-major slab [64 k][R cols]: R/8 chunks per k-row, permuted in pairs (a
// transposed read covers 16 columns = one chunk pair) by a k-row-dependent
// amount so that the 16 k-rows one read instruction touches land on
// distinct banks.  R = 256 (16 pairs): rotation of the pairs.  R = 192
// (12 pairs, where a rotation would wrap unevenly): XOR inside aligned
// blocks of 4 pairs.
__device__ __forceinline__ int rot_mnmaj(int krow) { return (krow & 3) + 4 * ((krow >> 3) & 1); }
__device__ __forceinline__ int xor_mnmaj(int krow)
{
    return ((krow >> 1) & 1) + 2 * ((krow & 1) ^ ((krow >> 3) & 1));
}

template <int R>
__device__ __forceinline__ int mn_phys_chunk(int krow, int logical_chunk)
{
    int pair = logical_chunk >> 1;
    if constexpr (R == 256) {
        pair += rot_mnmaj(krow);
        if (pair >= 16) pair -= 16;
    } else {
        pair ^= xor_mnmaj(krow);
    }
    return 2 * pair + (logical_chunk & 1);
}

template <int R>
__device__ __forceinline__ int mn_logical_chunk(int krow, int phys_chunk)
{
    int pair = phys_chunk >> 1;
    if constexpr (R == 256) {
        pair -= rot_mnmaj(krow);
        if (pair < 0) pair += 16;
    } else {
        pair ^= xor_mnmaj(krow);
    }
    return 2 * pair + (phys_chunk & 1);
}

// Loads of one R x 64 operand slab (R = 256 or 192 rows of M or N) into an
// LDS stage.  The slab is R * 8 chunks of 16 bytes; instruction j of wave w
// fills chunks [(w * kPerWave + j) * 64, +64), one per lane, contiguously.
template <bool KMAJ, int R>
struct SlabDma {
    static constexpr int kPerWave = R / 8 / kWaves;
    static_assert(kPerWave * kWaves * 8 == R, "slab does not split evenly over the waves");
    // Byte offsets of this lane for slab 0.  Out-of-range elements are given
    // the offset 0x80000000, beyond any operand (< 2^31 bytes), so the buffer
    // descriptor returns zeros for them; only the per-lane offset is relied on
    // for that, never the scalar one.
    static constexpr uint32_t kInvalid = 0x80000000u;
    uint32_t voff[kPerWave];
    int krow[kPerWave];        // MN-major: k-row of the slab this lane loads
    uint32_t kstep;            // bytes to advance one slab along K
    int64_t K;

    __device__ __forceinline__ void init(int wave, int lane, int64_t r0, int64_t ld,
                                         int64_t extent, int64_t K_)
    {
        K = K_;
#pragma unroll
        for (int j = 0; j < kPerWave; ++j) {
            const int linear = (wave * kPerWave + j) * 64 + lane;
            if (KMAJ) {
                const int row = linear >> 3;
                const int chunk = (linear & 7) ^ swz_kmaj(row);
                voff[j] = r0 + row < extent ? (uint32_t)(((r0 + row) * ld + chunk * 8) * 2)
                                            : kInvalid;
                krow[j] = 0;
            } else {
                krow[j] = linear / (R / 8);
                const int chunk = mn_logical_chunk<R>(krow[j], linear % (R / 8));
                voff[j] = r0 + chunk * 8 < extent ? (uint32_t)((krow[j] * ld + r0 + chunk * 8) * 2)
                                                  : kInvalid;
            }
        }
        kstep = KMAJ ? (uint32_t)(kBK * 2) : (uint32_t)(kBK * ld * 2);
    }

    // K-major: K is a multiple of the slab depth, so the slab offset (scalar)
    // keeps every in-range row inside the operand.  MN-major: the slab offset
    // is added per lane, and k-rows past K are invalidated.
    __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rsrc, bf16* slab, int wave,
                                          int kt) const
    {
#pragma unroll
        for (int j = 0; j < kPerWave; ++j) {
            bf16* dst = slab + (wave * kPerWave + j) * 64 * 8;
            if (KMAJ) {
                load_lds16(rsrc, dst, voff[j], (uint32_t)kt * kstep);
            } else {
                const bool ok = voff[j] != kInvalid && (int64_t)kt * kBK + krow[j] < K;
                load_lds16(rsrc, dst, ok ? voff[j] + (uint32_t)kt * kstep : kInvalid, 0u);
            }
        }
    }
};

// Fragment reads for one 32-wide k half (ks) of a slab: NF fragments of 16
// rows (M for A, N for B) x 32 k, 8 bf16 per lane.
template <bool KMAJ, int R, int NF>
__device__ __forceinline__ void read_frags(const bf16* slab, int wrow0, int ks, int lane,
                                           bf16x8 (&f)[NF])
{
    const int i = lane & 15, g = lane >> 4;
    if constexpr (KMAJ) {
        const int chunk = (ks * 4 + g) ^ swz_kmaj(i);
#pragma unroll
        for (int q = 0; q < NF; ++q) {
            const int row = wrow0 + q * 16 + i;
            f[q] = *reinterpret_cast<const bf16x8*>(slab + row * kBK + chunk * 8);
        }
    } else {
        // Lane 4e + c of each 16-lane group points at k-row e, columns
        // 4c..4c+3 of the fragment; the transposed read hands every lane four
        // consecutive k of its own column.
        const int krow0 = ks * 32 + g * 8 + (i >> 2);
#pragma unroll
        for (int q = 0; q < NF; ++q) {
            const int col = wrow0 + q * 16 + 4 * (i & 3);
            bf16x4 half[2];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int krow = krow0 + 4 * hh;
                const int chunk = mn_phys_chunk<R>(krow, col >> 3);
                const bf16* p = slab + krow * R + chunk * 8 + (col & 7);
                const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (TP_LDS i16x4*)((TP_LDS bf16*)p));
                half[hh] = __builtin_bit_cast(bf16x4, v);
            }
            f[q] = bf16x8{half[0][0], half[0][1], half[0][2], half[0][3],
                          half[1][0], half[1][1], half[1][2], half[1][3]};
        }
    }
}

template <int BN, bool A_KMAJ, bool B_KMAJ, Epi EPI, typename OutT>
__global__ __launch_bounds__(kThreads, 1) void gemm_tile_kernel(GemmArgs p, int tiles_m,
                                                                int tiles_n)
{
    constexpr int kWaveM = kBM / kWavesM;
    constexpr int kWaveN = BN / kWavesN;
    constexpr int kFragM = kWaveM / 16;
    constexpr int kFragN = kWaveN / 16;
    constexpr int kSlabA = kBM * kBK, kSlabB = BN * kBK;   // elements
    __shared__ __attribute__((aligned(1024))) bf16 smem[2][kSlabA + kSlabB];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / kWavesN, wn = wave % kWavesN;

    // XCD-aware tile order: the tiles of one XCD form a contiguous run of the
    // m-fastest tile sequence.
    const int ntiles = tiles_m * tiles_n;
    int tile = blockIdx.x;
    if (ntiles % kXcds == 0) tile = (tile % kXcds) * (ntiles / kXcds) + tile / kXcds;
    const int tm = tile % tiles_m, tn = tile / tiles_m;
    const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * BN;

    const bf16* A = static_cast<const bf16*>(p.A);
    const bf16* B = static_cast<const bf16*>(p.B);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (uint32_t)(p.M * p.K * 2));
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(B, (uint32_t)(p.N * p.K * 2));

    SlabDma<A_KMAJ, kBM> da;
    SlabDma<B_KMAJ, BN> db;
    da.init(wave, lane, m0, A_KMAJ ? p.K : p.M, p.M, p.K);
    db.init(wave, lane, n0, B_KMAJ ? p.K : p.N, p.N, p.K);

    f32x4 acc[kFragM][kFragN];
#pragma unroll
    for (int a = 0; a < kFragM; ++a)
#pragma unroll
        for (int b = 0; b < kFragN; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = (int)((p.K + kBK - 1) / kBK);
    bf16x8 fa[2][kFragM], fb[2][kFragN];
    const int wrow_a = wm * kWaveM, wrow_b = wn * kWaveN;

    if (nk > 0) {
        da.issue(ra, smem[0], wave, 0);
        db.issue(rb, smem[0] + kSlabA, wave, 0);
        __syncthreads();
        read_frags<A_KMAJ, kBM>(smem[0], wrow_a, 0, lane, fa[0]);
        read_frags<B_KMAJ, BN>(smem[0] + kSlabA, wrow_b, 0, lane, fb[0]);
    }

    // Per slab: read the second k half of the current stage, then start the
    // DMA of the next slab into the other stage.  All LDS reads of the
    // current stage precede the DMA in program order, so the wait for the
    // DMA (which the compiler places before the next LDS read) falls after
    // the 128 MFMAs of this slab instead of before them.
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        read_frags<A_KMAJ, kBM>(smem[cur], wrow_a, 1, lane, fa[1]);
        read_frags<B_KMAJ, BN>(smem[cur] + kSlabA, wrow_b, 1, lane, fb[1]);
        if (kt + 1 < nk) {
            da.issue(ra, smem[cur ^ 1], wave, kt + 1);
            db.issue(rb, smem[cur ^ 1] + kSlabA, wave, kt + 1);
        }
#pragma unroll
        for (int a = 0; a < kFragM; ++a)
#pragma unroll
            for (int b = 0; b < kFragN; ++b)
                acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[0][b], fa[0][a], acc[a][b],
                                                                     0, 0, 0);
#pragma unroll
        for (int a = 0; a < kFragM; ++a)
#pragma unroll
            for (int b = 0; b < kFragN; ++b)
                acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[1][b], fa[1][a], acc[a][b],
                                                                     0, 0, 0);
        // Keep the MFMAs above the barrier: its fence waits for the DMA.
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
        if (kt + 1 < nk) {
            read_frags<A_KMAJ, kBM>(smem[cur ^ 1], wrow_a, 0, lane, fa[0]);
            read_frags<B_KMAJ, BN>(smem[cur ^ 1] + kSlabA, wrow_b, 0, lane, fb[0]);
        }
    }

    // Epilogue: lane holds row (lane % 16) and columns 4 * (lane / 16) + 0..3
    // of every 16 x 16 fragment.
    const bf16* bias = static_cast<const bf16*>(p.bias);
    const bf16* aux = static_cast<const bf16*>(p.aux);
    bf16* save = static_cast<bf16*>(p.save);
    OutT* C = static_cast<OutT*>(p.C);
#pragma unroll
    for (int b = 0; b < kFragN; ++b) {
        const int64_t col = n0 + wrow_b + b * 16 + 4 * (lane >> 4);
        if (col >= p.N) continue;
        float bv[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (EPI == Epi::Bias || EPI == Epi::BiasGelu) {
            if (bias) {
                const bf16x4 t4 = *reinterpret_cast<const bf16x4*>(bias + col);
#pragma unroll
                for (int e = 0; e < 4; ++e) bv[e] = (float)t4[e];
            }
        }
#pragma unroll
        for (int a = 0; a < kFragM; ++a) {
            const int64_t row = m0 + wrow_a + a * 16 + (lane & 15);
            if (row >= p.M) continue;
            const int64_t off = row * p.N + col;
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = acc[a][b][e];
            if constexpr (EPI == Epi::Bias) {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] += bv[e];
            } else if constexpr (EPI == Epi::BiasGelu) {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] += bv[e];
                if (save)
                    *reinterpret_cast<bf16x4*>(save + off) =
                        bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = gelu_tanh(v[e]);
            } else if constexpr (EPI == Epi::DGelu) {
                const bf16x4 y4 = *reinterpret_cast<const bf16x4*>(aux + off);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] *= gelu_tanh_grad((float)y4[e]);
            }
            if constexpr (sizeof(OutT) == 4) {
                *reinterpret_cast<f32x4*>(C + off) = f32x4{v[0], v[1], v[2], v[3]};
            } else {
                *reinterpret_cast<bf16x4*>(C + off) =
                    bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
            }
        }
    }
}

constexpr int kCUs = 256;   // MI355X compute units

// Fraction of the chip's MFMA time that does useful work for a tile width:
// the tiles of the last partial wave leave CUs idle, and ragged tiles
// compute padding.
double tile_efficiency(int64_t M, int64_t N, int bn)
{
    const int64_t tm = (M + kBM - 1) / kBM, tn = (N + bn - 1) / bn;
    const int64_t tiles = tm * tn;
    const int64_t waves = (tiles + kCUs - 1) / kCUs;
    return (double)(M * N) / ((double)waves * kCUs * kBM * bn);
}

int pick_bn(int64_t M, int64_t N)
{
    return tile_efficiency(M, N, 192) > tile_efficiency(M, N, 256) + 1e-9 ? 192 : 256;
}

template <int BN, bool AK, bool BK, Epi E, typename O>
hipError_t launch_bn(const GemmArgs& p, hipStream_t stream)
{
    const int tm = (int)((p.M + kBM - 1) / kBM);
    const int tn = (int)((p.N + BN - 1) / BN);
    hipLaunchKernelGGL((gemm_tile_kernel<BN, AK, BK, E, O>), dim3((unsigned)(tm * tn)),
                       dim3(kThreads), 0, stream, p, tm, tn);
    return hipGetLastError();
}

template <bool AK, bool BK, Epi E, typename O>
hipError_t launch(const GemmArgs& p, hipStream_t stream)
{
    if (pick_bn(p.M, p.N) == 192) return launch_bn<192, AK, BK, E, O>(p, stream);
    return launch_bn<256, AK, BK, E, O>(p, stream);
}

}  // namespace

bool gemm_tile_supported(const GemmArgs& p, Layout layout)
{
    if (p.M < kBM || p.N < 192) return false;
    // A K-major operand must not run past the end of a row inside a slab.
    if (layout != Layout::TN && p.K % kBK != 0) return false;
    const int64_t lim = (int64_t(1) << 31) - 1;
    return p.M * p.K * 2 <= lim && p.N * p.K * 2 <= lim;
}

hipError_t gemm_tile(const GemmArgs& p, Layout layout, Epi epi, Elt out, hipStream_t stream)
{
    switch (layout) {
    case Layout::NN:
        if (epi == Epi::BiasGelu) {
            if (out == Elt::BF16) return launch<true, false, Epi::BiasGelu, bf16>(p, stream);
            return launch<true, false, Epi::BiasGelu, float>(p, stream);
        }
        if (epi == Epi::Bias) {
            if (out == Elt::BF16) return launch<true, false, Epi::Bias, bf16>(p, stream);
            return launch<true, false, Epi::Bias, float>(p, stream);
        }
        if (out == Elt::BF16) return launch<true, false, Epi::Store, bf16>(p, stream);
        return launch<true, false, Epi::Store, float>(p, stream);
    case Layout::NT:
        if (epi == Epi::DGelu) {
            if (out == Elt::BF16) return launch<true, true, Epi::DGelu, bf16>(p, stream);
            return launch<true, true, Epi::DGelu, float>(p, stream);
        }
        if (out == Elt::BF16) return launch<true, true, Epi::Store, bf16>(p, stream);
        return launch<true, true, Epi::Store, float>(p, stream);
    case Layout::TN:
        return launch<false, false, Epi::Store, float>(p, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace tpmlp
