// mma_tile.hpp -- one work-group tile of C^T = A B^T for two bf16 operands
// stored row-major with the contraction dimension contiguous (A [N][K],
// B [M][K]), on v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
//
// Both operands stream through LDS with direct global->LDS loads
// (global_load_lds_dwordx4, 1 KB per wave instruction) in a ring of SLOTS
// stages of KC elements along K.  The 16-byte chunks of a row slice are
// XOR-swizzled so the fragment reads (32 rows x one chunk per half-wave)
// hit distinct banks.  A's rows are the MFMA's M side: after the call, lane
// l of wave (wn, wm) holds in acc[x][y][e] the dot product of B row
// (wm * TM + y) * 32 + l % 32 (of the tile's B rows) with A row
// (wn * TN + x) * 32 + (e / 4) * 8 + (l / 32) * 4 + e % 4 (of the tile's A
// rows) -- a lane owns one B row and 16 A rows per 32-tile.
#pragma once

#include "common.hpp"

namespace wedlm {

// Tile shape: NT rows of A x MT rows of B per work-group of NW waves, WN
// along A x NW/WN along B, K in stages of KC, SLOTS stages of LDS (SLOTS - 1
// in flight beyond the one computed).
template <int NT_, int MT_, int KC_, int SLOTS_, int WN_, int NW_ = 8>
struct TileCfg {
    static constexpr int NW = NW_;
    static constexpr int NT = NT_, MT = MT_, KC = KC_, SLOTS = SLOTS_, WN = WN_, WM = NW_ / WN_;
    static constexpr int AHEAD = SLOTS - 1;
    static constexpr int RB = KC * 2;                 // bytes of one row in a stage
    static constexpr int CPR = KC / 8;                // 16-byte chunks per row
    static constexpr int RPI = 1024 / RB;             // rows per 1 KB wave load
    static constexpr int ABYTES = NT * RB, BBYTES = MT * RB, SLOTB = ABYTES + BBYTES;
    static constexpr int LPS = (NT + MT) / RPI / NW;  // DMA instructions per wave per stage
    static constexpr int TN = NT / WN / 32, TM = MT / WM / 32;   // 32-tiles per wave
    static_assert(LPS * RPI * NW == NT + MT, "a stage must split into whole wave loads");
    static_assert(NT % RPI == 0 && TN >= 1 && TM >= 1 && CPR >= 2, "tile shape");
    static_assert(SLOTS * SLOTB <= 160 * 1024 - 4096, "LDS");
    static_assert(MT <= 64 * NW, "one thread per B row for row lists");
    // chunk c of row r sits at c ^ g(r): 16 consecutive rows (one half-wave
    // reading one chunk each) land on 16 distinct 16-byte bank groups
    __device__ static int swz(int row, int c) { return c ^ ((row / (256 / RB)) & (CPR - 1)); }
    __device__ static int wave_n() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) % WN; }
    __device__ static int wave_m() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) / WN; }
};

template <int N>
__device__ __forceinline__ void tile_wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
__device__ __forceinline__ void tile_block_sync() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// acc = A[n0 .. n0+NT) . B[rows]^T over K elements (a multiple of KC) of
// rows ld elements long (arows(n) and B point at the first element of the
// K range of their row).  A rows at or past n_lim repeat row n_lim - 1 (the
// caller ignores their results); B rows are s_rows[0 .. MT) (LDS, set and
// synchronised by the caller), of which the first m_valid matter: a wave
// whose B rows all lie past them leaves its acc at zero.  s_ring: C::SLOTS * C::SLOTB bytes of LDS.
// Ends with a barrier-free ring: the caller synchronises before reusing
// s_ring.
// A row addresses: row n of a single matrix of `rowbytes`-long rows.
struct PlainRows {
    const char* A;
    size_t rowbytes;
    __device__ const char* operator()(int n) const { return A + (size_t)n * rowbytes; }
};

// A rows stacked from up to three matrices with the same row length: rows
// [0, n1) of p0, then [n1, n2) of p1, then the rest of p2.
struct StackedRows {
    const char* p0;
    const char* p1;
    const char* p2;
    int n1, n2;
    size_t rowbytes;
    __device__ const char* operator()(int n) const {
        return n < n1 ? p0 + (size_t)n * rowbytes
                      : (n < n2 ? p1 + (size_t)(n - n1) * rowbytes : p2 + (size_t)(n - n2) * rowbytes);
    }
};

template <class C, class ARows>
__device__ __forceinline__ void tile_mma_rows(const ARows arows, int n0, int n_lim, const char* Bm, const int* s_rows,
                                         int K, int ld, char* s_ring, f32x16 (&acc)[C::TN][C::TM],
                                         int m_valid = C::MT) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ns = K / C::KC;
    const size_t rowbytes = (size_t)ld * 2;

    // DMA sources of this lane: instruction q of a stage loads RPI row slices
    // (A rows for q < NT/RPI, then B rows); the lane that fills LDS chunk
    // (row, p) reads global chunk swz(row, p).
    // (the LDS offset of instruction q is q KB either way: the A rows fill
    // the first ABYTES = NT/RPI KB of a slot, the B rows follow)
    const char* gsrc[C::LPS];
#pragma unroll
    for (int u = 0; u < C::LPS; ++u) {
        const int q = w * C::LPS + u;
        const int p = lane % C::CPR;
        if (q < C::NT / C::RPI) {
            const int row = q * C::RPI + lane / C::CPR;
            const int n = min(n0 + row, n_lim - 1);
            gsrc[u] = arows(n) + C::swz(row, p) * 16;
        } else {
            const int m = (q - C::NT / C::RPI) * C::RPI + lane / C::CPR;
            gsrc[u] = Bm + (size_t)s_rows[m] * rowbytes + C::swz(m, p) * 16;
        }
    }
    static_assert(C::ABYTES == C::NT / C::RPI * 1024, "A rows fill whole 1 KB loads");
    auto issue = [&](int st) {
        char* slot = s_ring + (st % C::SLOTS) * C::SLOTB + w * C::LPS * 1024;
#pragma unroll
        for (int u = 0; u < C::LPS; ++u)
            __builtin_amdgcn_global_load_lds(
                (const void*)(gsrc[u] + (size_t)st * C::RB),
                (__attribute__((address_space(3))) void*)(reinterpret_cast<uintptr_t>(slot + u * 1024)), 16, 0, 0);
    };

    const int wn = w % C::WN, wm = w / C::WN;
    const int hl = lane >> 5, col = lane & 31;
    int arow[C::TN], brow[C::TM];
#pragma unroll
    for (int t = 0; t < C::TN; ++t) arow[t] = (wn * C::TN + t) * 32 + col;
#pragma unroll
    for (int t = 0; t < C::TM; ++t) brow[t] = (wm * C::TM + t) * 32 + col;
#pragma unroll
    for (int x = 0; x < C::TN; ++x)
#pragma unroll
        for (int y = 0; y < C::TM; ++y)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[x][y][e] = 0.f;

    // A wave whose B rows all lie at or past m_valid (a partly used row
    // group) only loads and synchronises: its results would be discarded,
    // and leaving the MFMA pipe to the other wave of its SIMD speeds that one
    // up.  The flag is wave-uniform.
    const bool active = wm * C::TM * 32 < m_valid;
    const int npro = ns < C::AHEAD ? ns : C::AHEAD;
    for (int st = 0; st < npro; ++st) issue(st);
    if (!active) {
        // the same waits, barriers and loads as the compute loop below
        for (int st = 0; st < ns; ++st) {
            switch (min(C::AHEAD - 1, ns - 1 - st)) {
                case 3: tile_wait_vm<3 * C::LPS>(); break;
                case 2: tile_wait_vm<2 * C::LPS>(); break;
                case 1: tile_wait_vm<C::LPS>(); break;
                default: tile_wait_vm<0>(); break;
            }
            tile_block_sync();
            if (st + C::AHEAD < ns) issue(st + C::AHEAD);
        }
        return;
    }
    for (int st = 0; st < ns; ++st) {
        // this wave's loads of stage st have landed (up to AHEAD-1 later
        // stages may still be in flight); the barrier publishes every wave's
        // part and frees the slot of stage st-1 for stage st+AHEAD
        switch (min(C::AHEAD - 1, ns - 1 - st)) {
            case 3: tile_wait_vm<3 * C::LPS>(); break;
            case 2: tile_wait_vm<2 * C::LPS>(); break;
            case 1: tile_wait_vm<C::LPS>(); break;
            default: tile_wait_vm<0>(); break;
        }
        tile_block_sync();
        if (st + C::AHEAD < ns) issue(st + C::AHEAD);
        const char* slot = s_ring + (st % C::SLOTS) * C::SLOTB;
#pragma unroll
        for (int s = 0; s < C::KC / 16; ++s) {
            bf16x8 af[C::TN], bf[C::TM];
#pragma unroll
            for (int t = 0; t < C::TN; ++t)
                af[t] = *reinterpret_cast<const bf16x8*>(slot + arow[t] * C::RB + C::swz(arow[t], 2 * s + hl) * 16);
#pragma unroll
            for (int t = 0; t < C::TM; ++t)
                bf[t] = *reinterpret_cast<const bf16x8*>(slot + C::ABYTES + brow[t] * C::RB +
                                                         C::swz(brow[t], 2 * s + hl) * 16);
#pragma unroll
            for (int x = 0; x < C::TN; ++x)
#pragma unroll
                for (int y = 0; y < C::TM; ++y)
                    acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[x], bf[y], acc[x][y], 0, 0, 0);
        }
    }
}

// The same over a single A matrix.
template <class C>
__device__ __forceinline__ void tile_mma(const char* A, int n0, int n_lim, const char* Bm, const int* s_rows, int K,
                                         int ld, char* s_ring, f32x16 (&acc)[C::TN][C::TM], int m_valid = C::MT) {
    tile_mma_rows<C>(PlainRows{A, (size_t)ld * 2}, n0, n_lim, Bm, s_rows, K, ld, s_ring, acc, m_valid);
}

}  // namespace wedlm
