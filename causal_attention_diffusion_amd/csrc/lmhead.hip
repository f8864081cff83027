// lmhead.hip -- the LM head of one WeDLM decode step fused with the select
// step's vocabulary statistics: logits z[r][v] = hidden[r] . lm_head[v]
// (bf16 operands, fp32 accumulation on MFMA) are folded into per-row
// (max, first argmax, S, T) as they leave the accumulators, so no logit is
// ever written to memory.
//
// Pages: WeDLM paper-summary page, "Method" (inference paragraph: each
// masked slot is scored by the entropy of the model's predictive
// distribution and filled with its most likely token) and TL;DR (the
// backbone is Qwen3-8B, whose output projection maps a 4096-wide hidden
// state to 151936 vocabulary logits).
//
// Four launches:
//   lmhead_rows   lists the masked rows of the window (only those are
//                 scored: filled slots need no prediction);
//   lmhead_stats  one work-group per (vocabulary tile of kLmNT entries,
//                 group of masked rows): C^T = W_tile H_group^T over the
//                 hidden size in stages, then the tile's statistics per row;
//   lmhead_merge  one wave per masked row merges its tiles' statistics;
//   commit_select_refill (select.hip) then runs commit / Eq. 11 / refill
//                 on the merged rows exactly as after vocab_stats.
//
// lmhead_stats streams both operands through LDS with direct global->LDS
// loads (global_load_lds_dwordx4, 1 KB per wave instruction) in a ring of
// stages, like the attention kernel.  The 16-byte chunks of a row slice are
// XOR-swizzled (LmCfg::swz) so the fragment reads (32 rows x one chunk per
// half-wave) hit distinct banks.  The MFMA is
// v_mfma_f32_32x32x16_bf16 with the vocabulary as its M side: a lane's 16
// accumulators are 16 vocabulary entries of one hidden row, so the row
// statistics are in-lane plus one exchange with lane ^ 32.
#include "kernels.hpp"
#include "stats.hpp"

namespace wedlm {

namespace {
constexpr int kNW = 8;   // waves per work-group

// Tile shape of lmhead_stats: NT vocabulary entries x MT masked rows per
// work-group, waves WN (vocabulary) x 8/WN (rows), the hidden size in stages
// of KC, SLOTS stages of LDS (SLOTS - 1 in flight beyond the one computed).
template <int NT_, int MT_, int KC_, int SLOTS_, int WN_>
struct LmCfg {
    static constexpr int NT = NT_, MT = MT_, KC = KC_, SLOTS = SLOTS_, WN = WN_, WM = kNW / WN_;
    static constexpr int AHEAD = SLOTS - 1;
    static constexpr int RB = KC * 2;                 // bytes of one row in a stage
    static constexpr int CPR = KC / 8;                // 16-byte chunks per row
    static constexpr int RPI = 1024 / RB;             // rows per 1 KB wave load
    static constexpr int ABYTES = NT * RB, BBYTES = MT * RB, SLOTB = ABYTES + BBYTES;
    static constexpr int LPS = (NT + MT) / RPI / kNW; // DMA instructions per wave per stage
    static constexpr int TN = NT / WN / 32, TM = MT / WM / 32;   // 32-tiles per wave
    static_assert(LPS * RPI * kNW == NT + MT, "a stage must split into whole wave loads");
    static_assert(NT % RPI == 0 && TN >= 1 && TM >= 1 && CPR >= 2, "tile shape");
    static_assert(SLOTS * SLOTB <= 160 * 1024 - 4096, "LDS");
    // chunk c of row r sits at c ^ g(r): 16 consecutive rows (one half-wave
    // reading one chunk each) land on 16 distinct 16-byte bank groups
    __device__ static int swz(int row, int c) { return c ^ ((row / (256 / RB)) & (CPR - 1)); }
};
// up to 128 window rows: the weights stream once, HBM-bound
using LmSmall = LmCfg<256, kLmMT, 64, 3, 4>;
// more rows: 256-row groups, waves of 128 x 64 (8 MFMAs per fragment set)
using LmLarge = LmCfg<256, 2 * kLmMT, 32, 4, 2>;

template <int N>
__device__ __forceinline__ void lm_wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
__device__ __forceinline__ void lm_block_sync() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
}  // namespace

// Compact list of the masked rows (global row b*W + j, increasing) and
// their count.  One work-group; a thread owns a contiguous run of rows.
__global__ __launch_bounds__(256) void lmhead_rows(LmheadArgs a) {
    __shared__ int s_cnt[256];
    const int t = threadIdx.x;
    const int per = (a.R + 255) / 256;
    const int r0 = t * per;
    int c = 0;
    for (int i = 0; i < per; ++i) {
        const int r = r0 + i;
        if (r < a.R && a.filled[r] == 0) ++c;
    }
    s_cnt[t] = c;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {   // inclusive scan
        const int v = t >= off ? s_cnt[t - off] : 0;
        __syncthreads();
        s_cnt[t] += v;
        __syncthreads();
    }
    int p = s_cnt[t] - c;
    for (int i = 0; i < per; ++i) {
        const int r = r0 + i;
        if (r < a.R && a.filled[r] == 0) a.rows[p++] = r;
    }
    if (t == 255) *a.count = s_cnt[255];
}

template <class C>
__global__ __launch_bounds__(512) void lmhead_stats(LmheadArgs a) {
    __shared__ __attribute__((aligned(1024))) char s_ring[C::SLOTS * C::SLOTB];
    __shared__ int s_rows[C::MT];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

    // Work-groups are handed to the 8 XCDs in turn.  The row groups of one
    // vocabulary tile get consecutive ids on the same XCD, so the tile's
    // weights come from HBM once and from that XCD's L2 for the others.
    const int i = blockIdx.x;
    const int xcd = i & 7, j = i >> 3;
    const int rg = j % a.nrg;
    const int vt = (j / a.nrg) * 8 + xcd;
    if (vt >= a.nvt) return;
    const int cnt = *a.count;
    const int c0 = rg * C::MT;
    if (c0 >= cnt) return;
    if (tid < C::MT) s_rows[tid] = a.rows[min(c0 + tid, cnt - 1)];   // rows past the count repeat a valid one
    __syncthreads();
    const int n0 = vt * C::NT;
    const int ns = a.Dm / C::KC;
    const size_t rowbytes = (size_t)a.Dm * 2;

    // DMA sources of this lane: instruction q of a stage loads RPI row slices
    // (weights for q < NT/RPI, then hidden rows); the lane that fills LDS
    // chunk (row, p) reads global chunk swz(row, p).
    const char* gsrc[C::LPS];
    uint32_t ldst[C::LPS];
#pragma unroll
    for (int u = 0; u < C::LPS; ++u) {
        const int q = w * C::LPS + u;
        const int p = lane % C::CPR;
        if (q < C::NT / C::RPI) {
            const int row = q * C::RPI + lane / C::CPR;
            const int n = min(n0 + row, a.V - 1);   // past the vocabulary: a valid row, masked below
            gsrc[u] = reinterpret_cast<const char*>(a.lm_head) + (size_t)n * rowbytes + C::swz(row, p) * 16;
            ldst[u] = q * 1024;
        } else {
            const int m = (q - C::NT / C::RPI) * C::RPI + lane / C::CPR;
            gsrc[u] = reinterpret_cast<const char*>(a.hidden) + (size_t)s_rows[m] * rowbytes + C::swz(m, p) * 16;
            ldst[u] = C::ABYTES + (q - C::NT / C::RPI) * 1024;
        }
    }
    auto issue = [&](int st) {
        char* slot = s_ring + (st % C::SLOTS) * C::SLOTB;
#pragma unroll
        for (int u = 0; u < C::LPS; ++u)
            __builtin_amdgcn_global_load_lds(
                (const void*)(gsrc[u] + (size_t)st * C::RB),
                (__attribute__((address_space(3))) void*)(reinterpret_cast<uintptr_t>(slot + ldst[u])), 16, 0, 0);
    };

    // wave (wn, wm): vocabulary rows wn*TN*32 .. (TN 32-tiles) x hidden rows
    // wm*TM*32 .. (TM 32-tiles)
    const int wn = w % C::WN, wm = w / C::WN;
    const int hl = lane >> 5, col = lane & 31;
    int arow[C::TN], brow[C::TM];
#pragma unroll
    for (int t = 0; t < C::TN; ++t) arow[t] = (wn * C::TN + t) * 32 + col;
#pragma unroll
    for (int t = 0; t < C::TM; ++t) brow[t] = (wm * C::TM + t) * 32 + col;
    f32x16 acc[C::TN][C::TM];
#pragma unroll
    for (int x = 0; x < C::TN; ++x)
#pragma unroll
        for (int y = 0; y < C::TM; ++y)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[x][y][e] = 0.f;

    const int npro = ns < C::AHEAD ? ns : C::AHEAD;
    for (int st = 0; st < npro; ++st) issue(st);
    for (int st = 0; st < ns; ++st) {
        // this wave's loads of stage st have landed (up to AHEAD-1 later
        // stages may still be in flight); the barrier publishes every wave's
        // part and frees the slot of stage st-1 for stage st+AHEAD
        switch (min(C::AHEAD - 1, ns - 1 - st)) {
            case 3: lm_wait_vm<3 * C::LPS>(); break;
            case 2: lm_wait_vm<2 * C::LPS>(); break;
            case 1: lm_wait_vm<C::LPS>(); break;
            default: lm_wait_vm<0>(); break;
        }
        lm_block_sync();
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

    // ---- statistics of this tile per hidden row
    lm_block_sync();   // every wave is done with the ring
    float4* s_stat = reinterpret_cast<float4*>(s_ring);   // [WN vocab waves][MT]
    constexpr int NZ = C::TN * 16;
#pragma unroll
    for (int y = 0; y < C::TM; ++y) {
        // the lane's NZ values in increasing vocabulary order: tile x, then
        // accumulator e (entry (e / 4) * 8 + hl * 4 + e % 4 of the 32-tile)
        float z[NZ];
#pragma unroll
        for (int x = 0; x < C::TN; ++x)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int v = n0 + (wn * C::TN + x) * 32 + (e >> 2) * 8 + hl * 4 + (e & 3);
                z[x * 16 + e] = v < a.V ? acc[x][y][e] : -INFINITY;
            }
        float bm = z[0];
#pragma unroll
        for (int k = 1; k < NZ; ++k) bm = fmaxf(bm, z[k]);
        Stat st{-INFINITY, 0x7fffffff, 0.f, 0.f};
        if (bm > -INFINITY) {
            int ba = 0x7fffffff;
#pragma unroll
            for (int k = NZ - 1; k >= 0; --k)   // backwards, so the first match wins
                if (z[k] == bm) ba = n0 + (wn * C::TN + (k >> 4)) * 32 + ((k & 15) >> 2) * 8 + hl * 4 + (k & 3);
            st.m = bm;
            st.a = ba;
        }
        float s = 0.f, t = 0.f;
#pragma unroll
        for (int k = 0; k < NZ; ++k) add_term(s, t, z[k], st.m);
        st.s = s;
        st.t = t;
        st = merge(st, shfl_xor_stat(st, 32));
        if (hl == 0)
            s_stat[wn * C::MT + (wm * C::TM + y) * 32 + col] = make_float4(st.m, __int_as_float(st.a), st.s, st.t);
    }
    __syncthreads();
    if (tid < C::MT && c0 + tid < cnt) {
        const float4 p0 = s_stat[tid];
        Stat o{p0.x, __float_as_int(p0.y), p0.z, p0.w};
#pragma unroll
        for (int k = 1; k < C::WN; ++k) {
            const float4 p = s_stat[k * C::MT + tid];
            o = merge(o, Stat{p.x, __float_as_int(p.y), p.z, p.w});
        }
        a.part[(size_t)(c0 + tid) * a.nvt + vt] = make_float4(o.m, __int_as_float(o.a), o.s, o.t);
    }
}

// One wave per masked row: merge its nvt tile statistics into one.
__global__ __launch_bounds__(64) void lmhead_merge(LmheadArgs a) {
    const int c = blockIdx.x;
    const int lane = threadIdx.x;
    const int cnt = *a.count;
    if (c >= cnt) return;
    const float4* pp = a.part + (size_t)c * a.nvt;
    Stat o{-INFINITY, 0x7fffffff, 0.f, 0.f};
    for (int v0 = 0; v0 < a.nvt; v0 += 4 * 64) {
        float4 x[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int v = v0 + q * 64 + lane;
            x[q] = v < a.nvt ? pp[v] : make_float4(0.f, 0.f, 0.f, 0.f);   // s == 0: empty
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) o = merge(o, Stat{x[q].x, __float_as_int(x[q].y), x[q].z, x[q].w});
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) o = merge(o, shfl_xor_stat(o, off));
    if (lane == 0) a.row_stat[a.rows[c]] = make_float4(o.m, __int_as_float(o.a), o.s, o.t);
}

hipError_t launch_lmhead(const LmheadArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(lmhead_rows, dim3(1), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned nvt8 = (unsigned)((a.nvt + 7) / 8);
    if (a.R <= LmSmall::MT) {
        LmheadArgs b = a;
        b.nrg = 1;
        hipLaunchKernelGGL(lmhead_stats<LmSmall>, dim3(8u * nvt8), dim3(512), 0, st, b);
    } else {
        LmheadArgs b = a;
        b.nrg = (a.R + LmLarge::MT - 1) / LmLarge::MT;
        hipLaunchKernelGGL(lmhead_stats<LmLarge>, dim3(8u * nvt8 * (unsigned)b.nrg), dim3(512), 0, st, b);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lmhead_merge, dim3((unsigned)a.R), dim3(64), 0, st, a);
    return hipGetLastError();
}

}  // namespace wedlm
