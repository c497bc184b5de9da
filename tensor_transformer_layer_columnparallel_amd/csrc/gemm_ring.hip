// Large-shape bf16 MFMA GEMM for gfx950: C[M,N] = epi( op(A)[M,K] * op(B)[K,N] ).
//
// Tiles of 256 x 192 outputs, one workgroup of NW = 8 waves (two per SIMD),
// each wave owning 256/WM x 192/(NW/WM) outputs, v_mfma_f32_16x16x32_bf16 with fp32
// accumulators and the B fragment in the first MFMA slot, so that each lane
// ends with four consecutive columns of one row.  Tiles are numbered so that
// consecutive workgroups (which the dispatcher spreads round-robin over the
// 8 XCDs) map to neighbouring tiles on the same XCD and share its L2.
//
// Operands are copied L2 -> LDS by buffer_load_dwordx4 ... lds (DMA, no VGPR
// staging) in 64-k blocks: a K-contiguous operand in units of 64 k (a unit
// row is one whole 128-byte line; a 32-k slab would fetch half lines, and
// half-line DMA moves half the bytes per cycle), an M/N-contiguous one in
// pairs of 32-k slabs (each slab row already whole lines).  A's units or
// pairs fill a ring of three (96 KiB), B's a ring of two (48 KiB).  The
// steps alternate: all of one A unit or pair at each even step (four loads
// per wave), all of one B unit or pair at each odd step (three), each two or
// three slabs before its first slab is read.
// The DMA is issued from inline assembly: the compiler's wait analysis cannot
// tell the buffers apart and would wait for the DMA just issued before any
// LDS read.  The waits are explicit instead.  Compute walks K in 32-k slabs;
// at an odd slab k every wave first
//   1. waits until its loads of A's and B's units or pairs for slabs k+1 and
//      k+2 have landed (the vector memory counter retires loads in issue
//      order; every wave issues the same number of DMA instructions per odd
//      and per even slab, so the counts are static) and until its own LDS
//      reads have returned;
//   2. passes a barrier: slabs k+1 and k+2 are in LDS for everybody and
//      nobody reads the buffers of slab k or earlier any more.
// An even slab needs neither (its reads and refills are covered by the
// barrier of the odd slab before): one barrier per 64 k.  At every slab the
// wave then, in four groups, each with the MFMAs of a share of the A
// fragments, (in all groups but the last) a share of the fragment reads, at
// raised wave priority, and a share of the DMA instructions, multiplies slab
// k (fragments read during slab k-1), reads the fragments of slab k+1 and
// refills a freed buffer.
// Spreading the memory instructions over the MFMAs keeps the waves of a SIMD
// from stalling together on a burst of loads while the matrix pipe idles.
// Loads of elements outside the operands (ragged M/N tails, k past K) use a
// per-lane offset of 2^31, beyond any operand, which the buffer descriptor
// turns into zeros without touching memory.
// Plain fp32 results are staged through the (then free) LDS ring so that the
// stores to HBM cover whole row segments (transposed on the way, for a
// result stored as C^T), written with non-temporal stores (the backward 2%
// faster; they measured slower for the stores below).  bf16 results are
// stored from the registers, eight consecutive columns per lane after a
// lane exchange between neighbouring fragments; the fp32 results of the
// GeLU epilogues four per lane.  The GeLU' epilogue can also sum its fp32
// results per column in a fixed order (one row of partials per 256-row
// block), the bias gradient's first step.
//
// LDS layouts (16-byte chunks permuted per row for conflict-free reads):
//   K-major 64-k unit [rows][64 k]: chunk c of row r at c ^ swz8(r), read
//                 with ds_read_b128;
//   MN-major slab [32 k][R cols]: chunk pairs rotated by k-row (R = 256, an A
//                 operand) or XORed in blocks of four (R = 192, a B operand);
//                 read with ds_read_b64_tr_b16 (lane i of a 16-lane group
//                 receives halfword i % 4 of the 8-byte pieces of lanes
//                 4e + i / 4).
#include <type_traits>

#include "common.h"
#include "epilogue.h"
#include "kernels.h"

namespace tpmlp {
namespace {

constexpr int kBM = 256;
constexpr int kBK = 32;
constexpr int kBN = 192;
constexpr int kABufs = 3;                   // A's ring: 64-k units or 32-k slab pairs
constexpr int kBBufs = 2;                   // B's ring (a power of two)
constexpr int kLead = 4;                    // DMA steps issued before the first slab
// Interleave groups per slab, and how many of them carry fragment reads.
// Only the first three of four groups carry reads, so the last group's
// MFMAs cover the latency of the last reads before the next wait (2-3%
// faster on the NN products than reads in all four groups, also at the odd
// slabs alone, which an even slab without a wait follows; reads in two
// groups or all up front were slower).  Within a group the reads follow the
// MFMAs (about 1% faster on the row-layer product and the backward than
// before them, the same on the column product) and the DMA instructions
// come last (0.6% faster on the backward than first).
constexpr int kGroups = 4;
constexpr int kReadGroups = 3;
// The fragment reads of the next slab issue at raised wave priority
// (s_setprio 1), so that a wave whose reads are due gets them out ahead of
// its SIMD partner's MFMAs: 3-4% faster on the row-layer product, 3% on the
// bias + GeLU product (which at the default priority ran best with two
// groups, reads in the first) and 1-1.5% on the backward.  Raising the
// MFMAs' or the DMA's priority instead measured no gain or slower.
constexpr int kXcds = 8;
constexpr int kCUs = 256;

// A tile configuration: BM x BN outputs per pipeline of NW waves, WM of them
// along M, KS pipelines per workgroup, at most OCC workgroups per CU.  Each
// pipeline has its own rings of kABufs 64-k units of A and kBBufs of B.
// With KS = 2 the workgroup's two pipelines compute the same tile over the
// two halves of K and at the end exchange halves of their sums, each
// finishing half of the tile's rows.
template <int BM_, int BN_, int NW_, int WM_, int OCC_, int KS_ = 1>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, NW = NW_, WM = WM_, OCC = OCC_, KS = KS_;
    static constexpr int ABytes = kABufs * BM * 64 * 2;
    static constexpr int BBytes = kBBufs * BN * 64 * 2;
    static_assert(KS == 1 || KS == 2, "one pipeline, or two over the halves of K");
};
// 256 x 192: every product of the GPT-3 shard splits into whole waves of 256
// CUs (256, 512 or 1536 tiles); 8 waves, 2 x 4 (NN, NT) or 4 x 2 (TN); rings
// of 96 + 48 KiB, one workgroup per CU.
using TileNN = TileCfg<256, 192, 8, 2, 1>;
using TileTN = TileCfg<256, 192, 8, 4, 1>;
// 128 x 96 for products with fewer 256 x 192 tiles than half the CUs (the
// 768 -> 3072 column layer: 64 tiles become 256, 20.6 -> 11.4 us): 4 waves of
// 64 x 48, rings of 48 + 24 KiB, up to two workgroups per CU (padding the
// LDS to one per CU measured 13% slower).  Each wave issues the same number
// of DMA instructions per step as in the large tile (4 for A's unit, 3 for
// B's), so the schedule and its waits are the same.
using TileSmall = TileCfg<128, 96, 4, 2, 2>;
// The same tile with K split between two pipelines of four waves in one
// workgroup (rings of 2 x 72 KiB, one workgroup per CU), for products with
// at most one 128 x 96 tile per CU: a lone four-wave workgroup spends about
// 500 cycles per 32-k slab on 192 cycles of MFMAs, its waits and barriers
// exposed with one wave per SIMD, and the second pipeline fills them while
// halving the slabs each one walks.  Each output is the first half's sum plus
// the second's; each pipeline finishes half of the tile's rows.
using TileSplit = TileCfg<128, 96, 4, 2, 1, 2>;

// Raw buffer descriptor (gfx9 family): base, stride 0, byte extent, word 3.
__device__ __forceinline__ i32x4 make_desc(const void* base, uint32_t bytes)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4 d;
    d[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    d[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
    d[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    d[3] = 0x00020000;
    return d;
}

// One 16-byte-per-lane DMA: lane l's bytes land at LDS byte address
// lds + 16 l (M0 holds lds).
__device__ __forceinline__ void dma16(i32x4 desc, uint32_t lds, uint32_t voff, uint32_t soff)
{
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(desc), "s"(soff)
                 : "memory", "m0");
}

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt out of range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

__device__ __forceinline__ void barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p)
{
    return (uint32_t)reinterpret_cast<uintptr_t>((TP_LDS const void*)p);
}

// Chunk permutation of K-major units (an XOR of row bits) for the fragment
// reads (lane l: row l % 16, chunk l / 16 (+ 4 for the unit's second slab),
// 16 bytes), chosen with a bank model; it runs at the full ds_read_b128 rate
// in a device probe and shows no bank-conflict cycles in the counters.
__device__ __forceinline__ int swz8(int row)
{
    return ((row >> 1) & 3) | (((row ^ (row >> 3)) & 1) << 2);
}

__device__ __forceinline__ int rot_mn(int krow) { return (krow & 3) + 4 * ((krow >> 3) & 1); }
__device__ __forceinline__ int xor_mn(int krow)
{
    return ((krow >> 1) & 1) + 2 * ((krow & 1) ^ ((krow >> 3) & 1));
}
// R = 96 (the small tile's B): the 6 pairs rotated by one for k-rows with
// bit 3 set, conflict-free for the transposing reads in the same bank model.
template <int R>
__device__ __forceinline__ int mn_phys(int krow, int chunk)
{
    static_assert(R == 256 || R == 192 || R == 96, "slab widths with a chunk permutation");
    int pair = chunk >> 1;
    if constexpr (R == 256) {
        pair += rot_mn(krow);
        if (pair >= 16) pair -= 16;
    } else if constexpr (R == 192) {
        pair ^= xor_mn(krow);
    } else {
        pair += (krow >> 3) & 1;
        if (pair >= 6) pair -= 6;
    }
    return 2 * pair + (chunk & 1);
}
template <int R>
__device__ __forceinline__ int mn_logical(int krow, int phys)
{
    int pair = phys >> 1;
    if constexpr (R == 256) {
        pair -= rot_mn(krow);
        if (pair < 0) pair += 16;
    } else if constexpr (R == 192) {
        pair ^= xor_mn(krow);
    } else {
        pair -= (krow >> 3) & 1;
        if (pair < 0) pair += 6;
    }
    return 2 * pair + (phys & 1);
}

constexpr uint32_t kInvalid = 0x80000000u;   // per-lane offset past any operand

// Bytes from an operand's first element to the end of its last one: R rows
// (M or N) by K, K-contiguous rows `ld` elements apart, or K rows of R
// elements `ld` apart.
__host__ __device__ __forceinline__ int64_t operand_bytes(bool kmajor, int64_t R, int64_t K,
                                                         int64_t ld)
{
    if (R <= 0 || K <= 0) return 0;
    return (kmajor ? (R - 1) * ld + K : (K - 1) * ld + R) * 2;
}

// DMA plan of a K-major 64-k unit stream of ROWS rows (A: 256, or the B of
// an NT product: 192) in a ring of BUFS units: ROWS rows x 128 bytes =
// ROWS / 8 instructions of 8 rows; wave w owns kPerUnit = ROWS / 8 / NW of
// them (instructions w * kPerUnit + q), all issued at one step.  Unit u
// covers k in [64u, 64u + 64); chunks past K, and units before the first,
// are invalidated per lane.
template <int NW, int ROWS, int BUFS>
struct UnitPlan {
    static_assert(ROWS % (8 * NW) == 0, "whole instructions per wave");
    static constexpr int kBufBytes = ROWS * 64 * 2;
    static constexpr int kPerUnit = ROWS / 8 / NW;    // instructions per wave and unit
    uint32_t voff[kPerUnit];
    int ulim[kPerUnit];   // units 0 <= u < ulim hold this lane's chunk inside K

    __device__ __forceinline__ void init(int wave, int lane, int64_t r0, int64_t ld,
                                         int64_t extent, int64_t K)
    {
#pragma unroll
        for (int q = 0; q < kPerUnit; ++q) {
            const int idx = wave * kPerUnit + q;
            const int row = idx * 8 + (lane >> 3);
            const int chunk = (lane & 7) ^ swz8(row);
            const bool ok = r0 + row < extent;
            voff[q] = ok ? (uint32_t)(((r0 + row) * ld + chunk * 8) * 2) : kInvalid;
            ulim[q] = ok ? (int)((K - chunk * 8 + 63) / 64) : 0;
        }
    }
    __device__ __forceinline__ void issue_q(int q, int wave, i32x4 desc, uint32_t ring_base,
                                            int unit) const
    {
        const uint32_t v =
            unit >= 0 && unit < ulim[q] ? voff[q] + (uint32_t)unit * 128u : kInvalid;
        const uint32_t buf = (uint32_t)(((unit % BUFS) + BUFS) % BUFS) * kBufBytes;
        const uint32_t lds = __builtin_amdgcn_readfirstlane(
            (int)(ring_base + buf + (uint32_t)(wave * kPerUnit + q) * 1024u));
        dma16(desc, lds, v, 0u);
    }
};

// DMA plan of an M/N-contiguous operand loaded two 32-k slabs at a time (B of
// the NN products, A and B of the TN products): R columns x 64 k = 2 R / 16
// instructions, kPer = 2 R / 16 / NW per wave (no filler slots).  A slab is
// [32 k][R] with its 16-byte chunks permuted per k-row (mn_phys); its
// instruction i fills chunks [64 i, 64 i + 64).  Pair v covers k-rows
// [64v, 64v + 64) and lives in slab buffers 2 (v mod BUFS) and
// 2 (v mod BUFS) + 1 of a ring of 2 BUFS slabs; k-rows past K, and pairs
// before the first, are invalidated per lane.
template <int NW, int R, int BUFS>
struct PairPlan {
    static constexpr int kSlabInstr = R / 16;
    static_assert((2 * kSlabInstr) % NW == 0, "whole instructions per wave");
    static constexpr int kPer = 2 * kSlabInstr / NW;
    static constexpr int kSlabBytes = R * kBK * 2;
    uint32_t voff[kPer];
    uint32_t dst[kPer];   // byte offset inside the pair's two slab buffers
    int krow[kPer];       // k-row inside the pair
    uint32_t kstep2;      // bytes from one pair to the next
    int64_t K;

    __device__ __forceinline__ void init(int wave, int lane, int64_t r0, int64_t ld,
                                         int64_t extent, int64_t K_)
    {
        K = K_;
        kstep2 = (uint32_t)(2 * kBK * ld * 2);
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int idx = wave * kPer + j;
            const int sl = idx / kSlabInstr, i = idx % kSlabInstr;
            const int linear = i * 64 + lane;
            const int kr = linear / (R / 8);
            const int chunk = mn_logical<R>(kr, linear % (R / 8));
            krow[j] = kr + kBK * sl;
            voff[j] = r0 + chunk * 8 < extent
                          ? (uint32_t)(((int64_t)krow[j] * ld + r0 + chunk * 8) * 2)
                          : kInvalid;
            dst[j] = (uint32_t)(sl * kSlabBytes + i * 1024);
        }
    }
    __device__ __forceinline__ void issue(int j, i32x4 desc, uint32_t ring_base, int pair) const
    {
        const bool ok = voff[j] != kInvalid && pair >= 0 && (int64_t)pair * 2 * kBK + krow[j] < K;
        const uint32_t v = ok ? voff[j] + (uint32_t)pair * kstep2 : kInvalid;
        const uint32_t buf = (uint32_t)(((pair % BUFS) + BUFS) % BUFS) * 2 * kSlabBytes;
        const uint32_t lds = __builtin_amdgcn_readfirstlane((int)(ring_base + buf + dst[j]));
        dma16(desc, lds, v, 0u);
    }
};

// One fragment of a 32-k slab: 16 rows (M for A, N for B) starting at row0,
// 8 bf16 per lane (lane l: row l % 16, k 8 (l / 16) .. 8 (l / 16) + 7).
// K-major 64-k unit buffer, slab half `half`.
__device__ __forceinline__ bf16x8 read_frag_k8(const bf16* buf, int row0, int half, int lane)
{
    const int i = lane & 15, g = lane >> 4;
    return *reinterpret_cast<const bf16x8*>(buf + (row0 + i) * 64 + ((4 * half + g) ^ swz8(i)) * 8);
}
// M/N-major 32-k slab buffer of R columns.
template <int R>
__device__ __forceinline__ bf16x8 read_frag_mn(const bf16* buf, int row0, int lane)
{
    const int i = lane & 15, g = lane >> 4;
    const int krow0 = g * 8 + (i >> 2);
    const int col = row0 + 4 * (i & 3);
    bf16x4 half[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int krow = krow0 + 4 * hh;
        const bf16* p = buf + krow * R + mn_phys<R>(krow, col >> 3) * 8 + (col & 7);
        const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TP_LDS i16x4*)((TP_LDS bf16*)p));
        half[hh] = __builtin_bit_cast(bf16x4, v);
    }
    return bf16x8{half[0][0], half[0][1], half[0][2], half[0][3],
                  half[1][0], half[1][1], half[1][2], half[1][3]};
}

// Writes a finished tile: lane holds row (lane % 16) and columns
// 4 * (lane / 16) + 0..3 of every 16 x 16 fragment of its wave's block
// (wave row wm, first rows/columns wrow_a/wrow_b of the tile).  Plain fp32
// results are staged through the LDS ring, which must no longer be read or
// written by any wave's loads.
template <class Cfg, Epi EPI, typename OutT>
__device__ __forceinline__ void store_tile(
    const GemmArgs& p, f32x4 (&acc)[Cfg::BM / Cfg::WM / 16][Cfg::BN / (Cfg::NW / Cfg::WM) / 16],
    bf16* smem, int64_t m0, int64_t n0, int tm, int wm, int wrow_a, int wrow_b, int lane,
    int a_lo = 0, int a_hi = Cfg::BM / Cfg::WM / 16)
{
    constexpr int NW = Cfg::NW, WM = Cfg::WM, BN = Cfg::BN, kBM = Cfg::BM;
    constexpr int kABytes = Cfg::ABytes, kBBytes = Cfg::BBytes;
    static_assert(EPI != Epi::DGelu || kBM == kGemmRingTileRows, "row blocks of GemmArgs::colsum");
    constexpr int kWavesM = WM, kWavesN = NW / WM;
    constexpr int kWaveN = BN / kWavesN;
    constexpr int kFragM = kBM / kWavesM / 16, kFragN = kWaveN / 16;

    const bf16* bias = static_cast<const bf16*>(p.bias);
    const bf16* aux = static_cast<const bf16*>(p.aux);
    OutT* C = static_cast<OutT*>(p.C);
    if constexpr (EPI == Epi::StoreT) {
        // C is [N][M]: column c of the tile is row n0 + c of C, the tile's
        // 256 rows contiguous in it.  Staged through LDS in two passes of
        // half the tile's columns, transposed on the way in (4-byte stores;
        // a pitch of kBM + 4 words puts the four column groups of a store on
        // distinct banks), then copied out as 16-byte chunks of whole rows.
        static_assert(sizeof(OutT) == 4, "transposed results are fp32");
        constexpr int kColsPass = BN / 2;
        constexpr int kPitchT = kBM + 4;   // words
        constexpr int kChunksRow = kBM / 4;
        static_assert(kColsPass * kPitchT * 4 <= kABytes + kBBytes, "staging exceeds the ring");
        static_assert(kColsPass % kWaveN == 0, "a wave's columns lie in one pass");
        float* stage = reinterpret_cast<float*>(smem);
        barrier();   // every wave's loads have landed and no wave reads the ring
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            const int c0 = pass * kColsPass;
            if (wrow_b >= c0 && wrow_b < c0 + kColsPass) {   // uniform per wave
#pragma unroll
                for (int a = 0; a < kFragM; ++a) {
                    const int r = wrow_a + a * 16 + (lane & 15);
#pragma unroll
                    for (int b = 0; b < kFragN; ++b)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int c = wrow_b + b * 16 + 4 * (lane >> 4) + e - c0;
                            stage[c * kPitchT + r] = acc[a][b][e];
                        }
                }
            }
            wait_lgkmcnt0();   // s_barrier itself does not wait for LDS stores
            barrier();
            for (int q = threadIdx.x; q < kColsPass * kChunksRow; q += 64 * NW) {
                const int row = q / kChunksRow, ch = q % kChunksRow;
                const int64_t gn = n0 + c0 + row, gm = m0 + (int64_t)ch * 4;
                if (gn < p.N && gm < p.M)   // M % 4 == 0: a chunk is all in or all out
                    __builtin_nontemporal_store(
                        *reinterpret_cast<const i32x4*>(stage + row * kPitchT + ch * 4),
                        reinterpret_cast<i32x4*>(C + gn * p.M + gm));
            }
            barrier();
        }
        return;
    }
    if constexpr (sizeof(OutT) == 4 && (EPI == Epi::Store || EPI == Epi::Bias)) {
        // Plain fp32 results (the row-layer partials and the backward's
        // gradients) go through LDS (the ring is free now) so that the stores
        // to HBM are whole 16-byte chunks of consecutive columns, one row
        // segment per group of lanes, instead of 16 rows x 64 bytes per store
        // instruction: 3-4% faster on those products.  (The bf16 outputs,
        // stored in 64-byte pieces of 16 rows, gain nothing from staging.)
        constexpr int kRowBytes = BN * 4;
        constexpr int kPitch = kRowBytes + 16;   // rows 16 bytes apart in bank space
        constexpr int kRows = kBM * kPitch <= kABytes + kBBytes ? kBM : kBM / 2;
        static_assert(kRows * kPitch <= kABytes + kBBytes, "staging exceeds the ring");
        constexpr int kChunks = kRows * (kRowBytes / 16);
        char* stage = reinterpret_cast<char*>(smem);
        barrier();   // every wave's loads have landed and no wave reads the ring
#pragma unroll
        for (int b = 0; b < kFragN; ++b) {
            const int64_t gcol = n0 + wrow_b + b * 16 + 4 * (lane >> 4);
            if constexpr (EPI == Epi::Bias) {
                if (bias && gcol < p.N) {
                    const bf16x4 t4 = *reinterpret_cast<const bf16x4*>(bias + gcol);
#pragma unroll
                    for (int a = 0; a < kFragM; ++a)
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[a][b][e] += (float)t4[e];
                }
            }
        }
#pragma unroll
        for (int r0 = 0; r0 < kBM; r0 += kRows) {
#pragma unroll
            for (int a = 0; a < kFragM; ++a) {
                const int row = wrow_a + a * 16 + (lane & 15) - r0;
                if (row < 0 || row >= kRows) continue;   // uniform per (wave, a)
#pragma unroll
                for (int b = 0; b < kFragN; ++b) {
                    const int col = wrow_b + b * 16 + 4 * (lane >> 4);
                    *reinterpret_cast<f32x4*>(stage + row * kPitch + col * 4) = acc[a][b];
                }
            }
            wait_lgkmcnt0();   // s_barrier itself does not wait for LDS stores
            barrier();
            for (int c = threadIdx.x; c < kChunks; c += 64 * NW) {
                const int row = c / (kRowBytes / 16), ch = c % (kRowBytes / 16);
                const int64_t grow = m0 + r0 + row, gcol = n0 + (int64_t)ch * 4;
                if (grow < p.M && gcol < p.N)
                    __builtin_nontemporal_store(
                        *reinterpret_cast<const i32x4*>(stage + row * kPitch + ch * 16),
                        reinterpret_cast<i32x4*>(C + grow * p.N + gcol));
            }
            barrier();
        }
        return;
    }
    bf16* save = static_cast<bf16*>(p.save);
    float cs[kFragN][4];   // DGelu: this lane's share of the tile's column sums
#pragma unroll
    for (int b = 0; b < kFragN; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) cs[b][e] = 0.f;
    if constexpr (sizeof(OutT) == 2) {
        // bf16 results leave in 16-byte pieces: for each pair of neighbouring
        // 16-column fragments b, b + 1, v_permlane16_swap exchanges fragment
        // b's values of lane rows 1 and 3 with fragment b + 1's of rows 0 and
        // 2, so that lane row g then holds eight consecutive columns
        // (fragment b + (g & 1), columns 8 (g >> 1) ..) and each store covers
        // 64 contiguous bytes of 16 rows instead of 32.  Every lane takes part
        // in the exchange; loads and stores outside the matrix are skipped.
        const int g = lane >> 4;
        float bv[kFragN][4];
#pragma unroll
        for (int b = 0; b < kFragN; ++b) {
            const int64_t col = n0 + wrow_b + b * 16 + 4 * g;
#pragma unroll
            for (int e = 0; e < 4; ++e) bv[b][e] = 0.f;
            if constexpr (EPI == Epi::Bias || EPI == Epi::BiasGelu) {
                if (bias && col < p.N) {
                    const bf16x4 t4 = *reinterpret_cast<const bf16x4*>(bias + col);
#pragma unroll
                    for (int e = 0; e < 4; ++e) bv[b][e] = (float)t4[e];
                }
            }
        }
        auto pack = [](float x0, float x1) {
            return (uint32_t)__builtin_bit_cast(uint16_t, (bf16)x0) |
                   ((uint32_t)__builtin_bit_cast(uint16_t, (bf16)x1) << 16);
        };
        // Stores one row of 16 x 16 fragments (w: packed pairs per fragment).
        auto store_row = [&](bf16* dst, uint32_t (&w)[kFragN][2], int64_t row) {
            const bool rowok = row < p.M;
#pragma unroll
            for (int b = 0; b + 1 < kFragN; b += 2) {
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const auto r = __builtin_amdgcn_permlane16_swap(w[b][h2], w[b + 1][h2], false,
                                                                    false);
                    w[b][h2] = r[0];
                    w[b + 1][h2] = r[1];
                }
                const int64_t col = n0 + wrow_b + (b + (g & 1)) * 16 + 8 * (g >> 1);
                if (rowok && col < p.N)   // N % 8 == 0: eight columns all in or all out
                    *reinterpret_cast<uint4*>(dst + row * p.N + col) =
                        uint4{w[b][0], w[b][1], w[b + 1][0], w[b + 1][1]};
            }
            if constexpr (kFragN % 2 == 1) {
                constexpr int b = kFragN - 1;
                const int64_t col = n0 + wrow_b + b * 16 + 4 * g;
                if (rowok && col < p.N)
                    *reinterpret_cast<uint2*>(dst + row * p.N + col) = uint2{w[b][0], w[b][1]};
            }
        };
#pragma unroll
        for (int a = 0; a < kFragM; ++a) {
            if (a < a_lo || a >= a_hi) continue;   // uniform per wave
            const int64_t row = m0 + wrow_a + a * 16 + (lane & 15);
            uint32_t hw[kFragN][2], yw[kFragN][2];
            // GeLU': the saved pre-activation comes in the same 16-byte
            // pieces and goes back to the fragments' layout through the same
            // exchange (it is its own inverse)
            uint32_t aw[kFragN][2];
            if constexpr (EPI == Epi::DGelu) {
                const bool rowok = row < p.M;
#pragma unroll
                for (int b = 0; b + 1 < kFragN; b += 2) {
                    const int64_t col = n0 + wrow_b + (b + (g & 1)) * 16 + 8 * (g >> 1);
                    uint4 q{0u, 0u, 0u, 0u};
                    if (rowok && col < p.N)
                        q = *reinterpret_cast<const uint4*>(aux + row * p.N + col);
                    const auto r0 = __builtin_amdgcn_permlane16_swap(q.x, q.z, false, false);
                    const auto r1 = __builtin_amdgcn_permlane16_swap(q.y, q.w, false, false);
                    aw[b][0] = r0[0];
                    aw[b + 1][0] = r0[1];
                    aw[b][1] = r1[0];
                    aw[b + 1][1] = r1[1];
                }
                if constexpr (kFragN % 2 == 1) {
                    constexpr int b = kFragN - 1;
                    const int64_t col = n0 + wrow_b + b * 16 + 4 * g;
                    uint2 q{0u, 0u};
                    if (rowok && col < p.N)
                        q = *reinterpret_cast<const uint2*>(aux + row * p.N + col);
                    aw[b][0] = q.x;
                    aw[b][1] = q.y;
                }
            }
#pragma unroll
            for (int b = 0; b < kFragN; ++b) {
                const int64_t col = n0 + wrow_b + b * 16 + 4 * g;
                const bool ok = row < p.M && col < p.N;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = acc[a][b][e];
                if constexpr (EPI == Epi::Bias) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] += bv[b][e];
                } else if constexpr (EPI == Epi::BiasGelu) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] += bv[b][e];
                    yw[b][0] = pack(v[0], v[1]);
                    yw[b][1] = pack(v[2], v[3]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = gelu_tanh(v[e]);
                } else if constexpr (EPI == Epi::DGelu) {
                    const bf16x4 y4 = __builtin_bit_cast(bf16x4, uint2{aw[b][0], aw[b][1]});
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        // the column sums add the products as computed, never
                        // fused with them into one multiply-add
#pragma clang fp contract(off)
                        v[e] *= gelu_tanh_grad((float)y4[e]);
                        if (ok) cs[b][e] += v[e];
                    }
                }
                hw[b][0] = pack(v[0], v[1]);
                hw[b][1] = pack(v[2], v[3]);
            }
            if constexpr (EPI == Epi::BiasGelu) {
                if (save) store_row(save, yw, row);
            }
            store_row(C, hw, row);
        }
    } else {   // fp32 results from registers (bias + GeLU, GeLU')
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
                    for (int e = 0; e < 4; ++e) {
#pragma clang fp contract(off)
                        v[e] *= gelu_tanh_grad((float)y4[e]);
                        cs[b][e] += v[e];
                    }
                }
                *reinterpret_cast<f32x4*>(C + off) = f32x4{v[0], v[1], v[2], v[3]};
            }
        }
    }
    if constexpr (EPI == Epi::DGelu) {
        if (p.colsum) {
            // Column sums of the tile's fp32 results (the bias gradient's
            // partials), in a fixed order: each lane's rows, then the 16
            // lanes that share a column (a butterfly; every lane ends with
            // the same value), then the wave rows in order.  Rows past M
            // were skipped above.
            float* red = reinterpret_cast<float*>(smem);   // [kWavesM][BN]
            barrier();   // no wave still reads the ring
#pragma unroll
            for (int b = 0; b < kFragN; ++b) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float v = cs[b][e];
#pragma unroll
                    for (int off = 1; off < 16; off <<= 1) v += __shfl_xor(v, off, 64);
                    if ((lane & 15) == 0)
                        red[wm * BN + wrow_b + b * 16 + 4 * (lane >> 4) + e] = v;
                }
            }
            wait_lgkmcnt0();
            barrier();
            const int c = threadIdx.x;
            if (c < BN && n0 + c < p.N) {
                float v = 0.f;
#pragma unroll
                for (int w = 0; w < kWavesM; ++w) v += red[w * BN + c];
                p.colsum[(int64_t)tm * p.N + n0 + c] = v;
            }
        }
    }
}

// The tile (tm, tn) this workgroup computes.  Tiles of all products are in
// one numbering, product-major; workgroups are remapped so that each XCD
// (the dispatcher sends workgroup w to XCD w mod 8) owns a contiguous run of
// tiles, which then lies in one product (one shard per XCD when eight shards
// are batched).  For a batch, p's operand pointers are moved to the
// workgroup's product.
template <typename OutT>
__device__ __forceinline__ void tile_of_block(GemmArgs& p, int tiles_m, int tiles_n, int group_m,
                                              int& tm, int& tn)
{
    const int per_product = tiles_m * tiles_n;
    const int ntiles = per_product * (int)p.batch;
    int tile = blockIdx.x;
    if (ntiles % kXcds == 0) tile = (tile % kXcds) * (ntiles / kXcds) + tile / kXcds;
    if (p.batch > 1) {
        const int64_t b = tile / per_product;
        tile -= (int)b * per_product;
        p.A = static_cast<const bf16*>(p.A) + b * p.sA;
        p.B = static_cast<const bf16*>(p.B) + b * p.sB;
        p.C = static_cast<OutT*>(p.C) + b * p.sC;
        if (p.bias) p.bias = static_cast<const bf16*>(p.bias) + b * p.sBias;
        if (p.save) p.save = static_cast<bf16*>(p.save) + b * p.sSave;
    }
    tm = tile % tiles_m;
    tn = tile / tiles_m;
    if (group_m > 0 && tiles_m % group_m == 0) {
        // Tiles in groups of group_m tile rows, column by column inside a
        // group, so that an XCD's run of tiles covers a group_m-row block.
        const int per_group = group_m * tiles_n;
        const int grp = tile / per_group, r = tile % per_group;
        tm = grp * group_m + r % group_m;
        tn = r / group_m;
    }
}

template <class Cfg, bool A_KMAJ, bool B_KMAJ, Epi EPI, typename OutT>
__global__ __launch_bounds__(64 * Cfg::NW * Cfg::KS, Cfg::OCC) void gemm_ring_kernel(GemmArgs p,
                                                                           int tiles_m,
                                                                           int tiles_n,
                                                                           int group_m)
{
    constexpr int NW = Cfg::NW, WM = Cfg::WM, BN = Cfg::BN, kBM = Cfg::BM;
    constexpr int kABytes = Cfg::ABytes, kBBytes = Cfg::BBytes;
    constexpr int kWavesM = WM, kWavesN = NW / WM;
    constexpr int kWaveM = kBM / kWavesM, kWaveN = BN / kWavesN;
    constexpr int kFragM = kWaveM / 16, kFragN = kWaveN / 16;
    // A: 64-k units (K-contiguous) or pairs of 32-k slabs (M-contiguous) in
    // a ring of three, all of one unit or pair at each even step; B likewise
    // (units for NT, slab pairs for NN and TN) in a ring of two at the odd
    // steps.  The steps alternate between A's loads and B's.
    using PlanAU = UnitPlan<NW, kBM, kABufs>;
    using PlanAP = PairPlan<NW, kBM, kABufs>;
    using PlanBU = UnitPlan<NW, BN, kBBufs>;
    using PlanBP = PairPlan<NW, BN, kBBufs>;
    static_assert(PlanAU::kBufBytes == 2 * PlanAP::kSlabBytes &&
                      PlanBU::kBufBytes == 2 * PlanBP::kSlabBytes,
                  "a unit and a slab pair take the same bytes");
    // DMA instructions per wave at even steps (A) and at odd steps (B).
    constexpr int kDmaEven = A_KMAJ ? PlanAU::kPerUnit : PlanAP::kPer;
    constexpr int kDmaOdd = B_KMAJ ? PlanBU::kPerUnit : PlanBP::kPer;
    constexpr int KS = Cfg::KS;
    // A workgroup of two pipelines ends with them exchanging halves of their
    // sums; only the bf16 register-path epilogue (no barrier, no
    // workgroup-wide loops) follows, each pipeline writing its half.
    static_assert(KS == 1 || ((EPI == Epi::Store || EPI == Epi::Bias || EPI == Epi::BiasGelu) &&
                              sizeof(OutT) == 2),
                  "split-K workgroups take the bf16 register-path epilogues");
    __shared__ __attribute__((aligned(1024))) bf16 smem[KS * (kABytes + kBBytes) / 2];

    const int lane = threadIdx.x & 63;
    const int wave_wg = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int half = wave_wg / NW;          // the pipeline (0 unless KS = 2)
    const int wave = wave_wg % NW;          // the wave inside its pipeline
    const int wm = wave / kWavesN, wn = wave % kWavesN;
    bf16* const sa = smem + half * ((kABytes + kBBytes) / 2);   // A ring
    bf16* const sb = sa + kABytes / 2;                          // B ring

    int tm, tn;
    tile_of_block<OutT>(p, tiles_m, tiles_n, group_m, tm, tn);
    const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * BN;

    const int64_t lda = p.lda ? p.lda : (A_KMAJ ? p.K : p.M);
    const int64_t ldb = p.ldb ? p.ldb : (B_KMAJ ? p.K : p.N);
    // The k range of this pipeline: all of K, or with two pipelines the
    // first kspan = ceil(K / 2) rounded up to a 64-k unit and the rest.
    // Both walk kspan (the same slabs, so the same barriers); the loads of
    // k past the range read zeros.
    int64_t kspan = p.K, k0 = 0, klen = p.K;
    if constexpr (KS == 2) {
        kspan = (p.K + 127) / 128 * 64;
        k0 = half * kspan;
        klen = p.K - k0 < kspan ? (p.K - k0 > 0 ? p.K - k0 : 0) : kspan;
    }
    const bf16* const A = static_cast<const bf16*>(p.A) + (A_KMAJ ? k0 : k0 * lda);
    const bf16* const Bp = static_cast<const bf16*>(p.B) + (B_KMAJ ? k0 : k0 * ldb);
    const i32x4 da = make_desc(A, (uint32_t)operand_bytes(A_KMAJ, p.M, klen, lda));
    const i32x4 db = make_desc(Bp, (uint32_t)operand_bytes(B_KMAJ, p.N, klen, ldb));
    PlanAU pau;
    PlanAP pap;
    if constexpr (A_KMAJ) pau.init(wave, lane, m0, lda, p.M, klen);
    else pap.init(wave, lane, m0, lda, p.M, klen);
    PlanBU pbu;
    PlanBP pbp;
    if constexpr (B_KMAJ) pbu.init(wave, lane, n0, ldb, p.N, klen);
    else pbp.init(wave, lane, n0, ldb, p.N, klen);
    const uint32_t a_base = lds_addr(sa), b_base = lds_addr(sb);

    const int wrow_a = wm * kWaveM, wrow_b = wn * kWaveN;
    f32x4 acc[kFragM][kFragN];
#pragma unroll
    for (int a = 0; a < kFragM; ++a)
#pragma unroll
        for (int b = 0; b < kFragN; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 fa[2][kFragM], fb[2][kFragN];

    // DMA instruction d of step vs (negative in the prologue).  Even vs: A's
    // unit or pair (vs + 4) / 2, into the buffer of (vs - 2) / 2, whose last
    // slab (vs - 1) was read during step vs - 2.  Odd vs: B's unit or pair
    // (vs + 3) / 2, into the buffer of (vs - 1) / 2, whose last slab (vs)
    // was read during step vs - 1.  Each lands two or three slabs before its
    // first slab is read.  The prologue issues steps -4 .. -1 (A's units or
    // pairs 0 and 1, B's 0 and 1); the waits only ever count the most recent
    // steps, so they are those of the main loop.
    auto dma_op = [&](int d, int vs) {
        if ((vs & 1) == 0) {
            if constexpr (A_KMAJ) pau.issue_q(d, wave, da, a_base, (vs + 4) >> 1);
            else pap.issue(d, da, a_base, (vs + 4) >> 1);
        } else {
            if constexpr (B_KMAJ) pbu.issue_q(d, wave, db, b_base, (vs + 3) >> 1);
            else pbp.issue(d, db, b_base, (vs + 3) >> 1);
        }
    };
    // The work of one slab is cut into kGroups groups, each holding (in this
    // order) the MFMAs of the A fragments a with a % kGroups == g, (for g <
    // kReadGroups) the fragment reads of the next slab with index %
    // kReadGroups == g and the DMA instructions d with d % kGroups == g, so
    // that the waves never stall on a burst of memory instructions while the
    // matrix pipe idles.
    static_assert(kFragM % kGroups == 0, "whole A fragments per group");
    auto read_group = [&](int g, int slab, int buf) {
#pragma unroll
        for (int a = g; a < kFragM; a += kReadGroups) {
            if constexpr (A_KMAJ)
                fa[buf][a] = read_frag_k8(sa + ((slab >> 1) % kABufs) * (kBM * 64),
                                          wrow_a + a * 16, slab & 1, lane);
            else
                fa[buf][a] = read_frag_mn<kBM>(sa + (slab % (2 * kABufs)) * (kBM * kBK),
                                               wrow_a + a * 16, lane);
        }
#pragma unroll
        for (int q = g; q < kFragN; q += kReadGroups) {
            if constexpr (B_KMAJ)
                fb[buf][q] = read_frag_k8(sb + ((slab >> 1) & (kBBufs - 1)) * (BN * 64),
                                          wrow_b + q * 16, slab & 1, lane);
            else
                fb[buf][q] = read_frag_mn<BN>(sb + (slab % (2 * kBBufs)) * (BN * kBK),
                                              wrow_b + q * 16, lane);
        }
    };
    auto mfma_group = [&](int g, int buf) {
#pragma unroll
        for (int a = g; a < kFragM; a += kGroups)
#pragma unroll
            for (int b = 0; b < kFragN; ++b)
                acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[buf][b], fa[buf][a],
                                                                    acc[a][b], 0, 0, 0);
    };
    // Slab kt: multiply slab kt (fragments read during the previous slab)
    // while reading the fragments of slab kt+1 and refilling the rings.  An
    // odd step first waits for its own loads of A's unit or pair and B's
    // unit or pair (kt+1)/2, issued at steps kt-3 and kt-2 (only the even
    // step kt-1 may stay outstanding), then passes a barrier that makes
    // every wave's loads of both slabs kt+1 and kt+2 visible and retires
    // every wave's reads up to step kt-1.  An even step needs neither: its
    // reads (slab kt+1, the second slab of the unit the odd step before made
    // visible) and its refill (A's buffer last read during step kt-2) are
    // covered by the barrier of step kt-1, and the odd step's refill (B's
    // buffer last read during step kt-1) by its own barrier.  One barrier per
    // 64 k instead of two.
    auto slab_step = [&](auto odd, int kt, int cbuf, int nbuf) {
        constexpr bool kOdd = decltype(odd)::value;
        if constexpr (kOdd) {
            wait_vmcnt<kDmaEven>();
            wait_lgkmcnt0();
            barrier();
        }
        constexpr int kSteps = kOdd ? kDmaOdd : kDmaEven;
#pragma unroll
        for (int g = 0; g < kGroups; ++g) {
            mfma_group(g, cbuf);
            if (g < kReadGroups) {
                __builtin_amdgcn_s_setprio(1);
                read_group(g, kt + 1, nbuf);
                __builtin_amdgcn_s_setprio(0);
            }
#pragma unroll
            for (int d = g; d < kSteps; d += kGroups) dma_op(d, kt);
            // A scheduling barrier closes each group, except in the NN
            // products: there the compiler's own placement of the transposing
            // B reads across groups is 2-3% faster (column and row products;
            // for the NT products it measured 0.6% slower).
            if constexpr (!(A_KMAJ && !B_KMAJ)) __builtin_amdgcn_sched_barrier(0);
        }
    };
    using Even = std::integral_constant<bool, false>;
    using Odd = std::integral_constant<bool, true>;

    const int nk = (int)((kspan + kBK - 1) / kBK);
    if (nk > 0) {
        static_assert(kLead == 4, "the prologue starts at an even (A) step");
#pragma unroll
        for (int vs = -kLead; vs < 0; ++vs) {
            constexpr int kDmaMax = kDmaOdd > kDmaEven ? kDmaOdd : kDmaEven;
            const int steps = (vs & 1) ? kDmaOdd : kDmaEven;
#pragma unroll
            for (int d = 0; d < kDmaMax; ++d)
                if (d < steps) dma_op(d, vs);
        }
        // Slab 0 came with steps -4 (A) and -3 (B): only steps -2 and -1 may
        // be outstanding.
        wait_vmcnt<kDmaEven + kDmaOdd>();
        barrier();
#pragma unroll
        for (int g = 0; g < kReadGroups; ++g) read_group(g, 0, 0);
        int kt = 0;
        for (; kt + 1 < nk; kt += 2) {
            slab_step(Even{}, kt, 0, 1);
            slab_step(Odd{}, kt + 1, 1, 0);
        }
        if (kt < nk) slab_step(Even{}, kt, 0, 1);
    }
    wait_vmcnt<0>();
    wait_lgkmcnt0();
    if constexpr (KS == 2) {
        // The two pipelines' sums of the same outputs meet through LDS
        // (48 KiB, in the rings that nobody reads any more): pipeline h keeps
        // the fragment rows a in [h kFragM / 2, (h + 1) kFragM / 2), sends the
        // others to the wave of the other pipeline that holds the same
        // outputs, adds what it receives (fp32 addition is commutative, so
        // both halves get first half + second half) and writes its rows.
        static_assert(kFragM % 2 == 0, "fragment rows split between the pipelines");
        static_assert(NW * kFragM * kFragN * 64 * 16 <= kABytes + kBBytes, "hand-over space");
        constexpr int kHalf = kFragM / 2;
        f32x4* const red = reinterpret_cast<f32x4*>(smem);
        // fragment rows [kKeep, kKeep + kHalf) stay, the others go (constant
        // offsets: the accumulators stay in registers)
        auto send = [&](auto keep) {
            constexpr int kSend = kHalf - decltype(keep)::value;
#pragma unroll
            for (int a = 0; a < kHalf; ++a)
#pragma unroll
                for (int b = 0; b < kFragN; ++b)
                    red[((wave * kFragM + kSend + a) * kFragN + b) * 64 + lane] = acc[kSend + a][b];
        };
        auto receive = [&](auto keep) {
            constexpr int kKeep = decltype(keep)::value;
#pragma unroll
            for (int a = 0; a < kHalf; ++a)
#pragma unroll
                for (int b = 0; b < kFragN; ++b) {
                    const f32x4 r = red[((wave * kFragM + kKeep + a) * kFragN + b) * 64 + lane];
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[kKeep + a][b][e] = acc[kKeep + a][b][e] + r[e];
                }
        };
        using Lo = std::integral_constant<int, 0>;
        using Hi = std::integral_constant<int, kHalf>;
        const int a_lo = half * kHalf;
        barrier();   // both pipelines are done with their rings
        if (half == 0) send(Lo{});
        else send(Hi{});
        wait_lgkmcnt0();   // s_barrier itself does not wait for LDS stores
        barrier();
        if (half == 0) receive(Lo{});
        else receive(Hi{});
        store_tile<Cfg, EPI, OutT>(p, acc, smem, m0, n0, tm, wm, wrow_a, wrow_b, lane, a_lo,
                                   a_lo + kHalf);
        return;
    }
    store_tile<Cfg, EPI, OutT>(p, acc, smem, m0, n0, tm, wm, wrow_a, wrow_b, lane);
}

template <class Cfg, bool AK, bool BK, Epi E, typename O>
hipError_t launch_cfg(const GemmArgs& p, hipStream_t stream)
{
    const int tm = (int)((p.M + Cfg::BM - 1) / Cfg::BM);
    const int tn = (int)((p.N + Cfg::BN - 1) / Cfg::BN);
    // Products with several waves of tiles walk an XCD's tiles in 4-row
    // groups: the weight gradients (six waves) about 4% faster, the two-wave
    // NN row-layer product about 2%.  For the one-wave NN product (the column
    // layer: 8 x 32 tiles) the groups give each XCD a 4 x 8 block of tiles
    // instead of 8 x 4, so its L2 fetches half of X and a quarter of W1
    // (503 MB from HBM in all instead of 553) at the same speed.  NT
    // products with one or two waves of tiles keep the plain order, which
    // measured as fast or faster for them.  Batched products give each XCD
    // one product's tiles for its 32 CUs, so they take the 4-row groups too.
    const int group_m = tm * tn > 2 * kCUs || !BK || p.batch > 1 ? 4 : 0;
    hipLaunchKernelGGL((gemm_ring_kernel<Cfg, AK, BK, E, O>),
                       dim3((unsigned)(tm * tn * p.batch)), dim3(64 * Cfg::NW * Cfg::KS), 0,
                       stream, p, tm, tn, group_m);
    return hipGetLastError();
}

// Eight waves per workgroup on 256 x 192 tiles.  Four waves on the same tile
// (one per SIMD, 256 x 48 or 128 x 96 outputs each) read less LDS per flop
// but measured about 35% slower: with one wave per SIMD nothing covers a
// wave's own waits.  Products with a K-contiguous A and a forward epilogue
// run on 128 x 96 tiles instead:
//  - on two K-split pipelines per workgroup when one product has no more
//    128 x 96 tiles than CUs, K has at least four 64-k units and the results
//    are bf16 (stored from registers).  This depends on the product alone, not on the
//    batch: the split adds each output's k range in another order, and a
//    batch must give the same bits as its products launched one by one;
//  - otherwise on two workgroups of four waves per CU when the launch would
//    have fewer 256 x 192 tiles than half the CUs (the same k order as the
//    large tiles).
template <bool AK, bool BK, Epi E, typename O>
hipError_t launch(const GemmArgs& p, hipStream_t stream)
{
    if constexpr (AK && (E == Epi::Store || E == Epi::Bias || E == Epi::BiasGelu)) {
        if constexpr (sizeof(O) == 2) {
            const int64_t small = ((p.M + TileSmall::BM - 1) / TileSmall::BM) *
                                  ((p.N + TileSmall::BN - 1) / TileSmall::BN);
            if (small <= kCUs && p.K >= 256) return launch_cfg<TileSplit, AK, BK, E, O>(p, stream);
        }
        const int64_t tiles = ((p.M + kBM - 1) / kBM) * ((p.N + kBN - 1) / kBN) * p.batch;
        if (tiles < kCUs / 2) return launch_cfg<TileSmall, AK, BK, E, O>(p, stream);
    }
    return launch_cfg<std::conditional_t<AK, TileNN, TileTN>, AK, BK, E, O>(p, stream);
}

}  // namespace

bool gemm_ring_supported(const GemmArgs& p, Layout layout)
{
    if (p.M < kBM || p.N < 192) return false;
    // M/N-major operands are loaded and masked in 8-element chunks.
    if (p.N % 8 != 0 || (layout == Layout::TN && p.M % 8 != 0)) return false;
    // A K-major operand must not run past the end of a row inside a slab.
    if (layout != Layout::TN && p.K % kBK != 0) return false;
    const int64_t lim = (int64_t(1) << 31) - 1;
    if (p.batch < 1 || (int64_t)((p.M + kBM - 1) / kBM) * ((p.N + kBN - 1) / kBN) * p.batch >
                           (int64_t(1) << 30))
        return false;
    const bool ak = layout != Layout::TN, bk = layout == Layout::NT;
    const int64_t lda = p.lda ? p.lda : (ak ? p.K : p.M);
    const int64_t ldb = p.ldb ? p.ldb : (bk ? p.K : p.N);
    if (lda < (ak ? p.K : p.M) || ldb < (bk ? p.K : p.N)) return false;
    return operand_bytes(ak, p.M, p.K, lda) <= lim && operand_bytes(bk, p.N, p.K, ldb) <= lim;
}

hipError_t gemm_ring(const GemmArgs& p, Layout layout, Epi epi, Elt out, hipStream_t stream)
{
    if (p.batch > 1 && epi != Epi::Store && epi != Epi::Bias && epi != Epi::BiasGelu)
        return hipErrorInvalidValue;
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
        if (epi == Epi::StoreT) {
            // stored in 16-byte chunks of 4 consecutive rows
            if (out != Elt::F32 || p.M % 4 != 0) return hipErrorInvalidValue;
            return launch<true, false, Epi::StoreT, float>(p, stream);
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
