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
// lmhead_stats runs the tile contraction of mma_tile.hpp (both operands
// streamed through LDS by direct global->LDS loads) with the vocabulary as
// the MFMA's M side: a lane's 16 accumulators are 16 vocabulary entries of
// one hidden row, so the row statistics are in-lane plus one exchange with
// lane ^ 32.
#include "kernels.hpp"
#include "mma_tile.hpp"
#include "stats.hpp"

namespace wedlm {

// 256 vocabulary entries x 128 masked rows per work-group, waves of 64 x 64,
// K in stages of 64 (whole 128-byte lines of every row).  A 256 x 256 tile
// in stages of 32 moves fewer bytes per flop but fetches each line in two
// halves, and measured slower at every window size tried.
using LmTile = TileCfg<256, kLmMT, 64, 3, 4>;

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
__global__ __launch_bounds__(64 * C::NW) void lmhead_stats(LmheadArgs a) {
    __shared__ __attribute__((aligned(1024))) char s_ring[C::SLOTS * C::SLOTB];
    __shared__ int s_rows[C::MT];
    const int tid = threadIdx.x;
    const int lane = tid & 63;

    // Work-groups are handed to the 8 XCDs in turn.  The row groups of one
    // vocabulary tile get consecutive ids on the same XCD, so the tile's
    // weights come from HBM once and from that XCD's L2 for the others.
    // Only the row groups that hold masked rows take ids (the count is
    // device state; the grid is sized for every row): the active groups of a
    // tile are consecutive and the unused ids come last.  Interleaving the
    // unused ids with the active ones let the tiles' work-groups drift apart
    // in time, and a weight line lives in L2 for only microseconds here.
    const int i = blockIdx.x;
    const int xcd = i & 7, j = i >> 3;
    const int cnt = *a.count;
    const int na = min(a.nrg, (cnt + C::MT - 1) / C::MT);   // row groups with masked rows
    if (na <= 0) return;
    const int rg = j % na;
    const int vt = (j / na) * 8 + xcd;
    if (vt >= a.nvt) return;
    const int c0 = rg * C::MT;
    if (tid < C::MT) s_rows[tid] = a.rows[min(c0 + tid, cnt - 1)];   // rows past the count repeat a valid one
    __syncthreads();
    const int n0 = vt * C::NT;
    const int wn = C::wave_n(), wm = C::wave_m();
    const int hl = lane >> 5, col = lane & 31;
    f32x16 acc[C::TN][C::TM];
    tile_mma<C>(reinterpret_cast<const char*>(a.lm_head), n0, a.V, reinterpret_cast<const char*>(a.hidden), s_rows,
                a.Dm, a.Dm, s_ring, acc, cnt - c0);

    // ---- statistics of this tile per hidden row
    tile_block_sync();   // every wave is done with the ring
    float4* s_stat = reinterpret_cast<float4*>(s_ring);   // [WN vocab waves][MT]
#pragma unroll
    for (int y = 0; y < C::TM; ++y) {
        // the lane's values in increasing vocabulary order, one 32-tile (16
        // accumulators: entry (e / 4) * 8 + hl * 4 + e % 4) at a time
        Stat st{-INFINITY, 0x7fffffff, 0.f, 0.f};
#pragma unroll
        for (int x = 0; x < C::TN; ++x) {
            const int v0 = n0 + (wn * C::TN + x) * 32 + hl * 4;
            float z[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) z[e] = v0 + (e >> 2) * 8 + (e & 3) < a.V ? acc[x][y][e] : -INFINITY;
            float bm = z[0];
#pragma unroll
            for (int e = 1; e < 16; ++e) bm = fmaxf(bm, z[e]);
            if (bm > st.m) {
                int ba = 0x7fffffff;
#pragma unroll
                for (int e = 15; e >= 0; --e)   // backwards, so the first match wins
                    if (z[e] == bm) ba = v0 + (e >> 2) * 8 + (e & 3);
                raise_max(st, bm, ba);
            }
            float s = 0.f, t = 0.f;
#pragma unroll
            for (int e = 0; e < 16; ++e) add_term(s, t, z[e], st.m);
            st.s += s;
            st.t += t;
        }
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
    LmheadArgs b = a;
    b.nrg = (a.R + LmTile::MT - 1) / LmTile::MT;
    hipLaunchKernelGGL(lmhead_stats<LmTile>, dim3(8u * nvt8 * (unsigned)b.nrg), dim3(64 * LmTile::NW), 0, st, b);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lmhead_merge, dim3((unsigned)a.R), dim3(64), 0, st, a);
    return hipGetLastError();
}

}  // namespace wedlm
