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
//                 group of kLmMT masked rows): C^T = W_tile H_group^T over
//                 the hidden size in stages of kLmKC, then the tile's
//                 statistics per row;
//   lmhead_merge  one wave per masked row merges its tiles' statistics;
//   commit_select_refill (select.hip) then runs commit / Eq. 11 / refill
//                 on the merged rows exactly as after vocab_stats.
//
// lmhead_stats streams both operands through LDS with direct global->LDS
// loads (global_load_lds_dwordx4, 1 KB per wave instruction) in a ring of
// kAhead+1 stages, like the attention kernel.  Row slices are 128 bytes;
// the 16-byte chunk c of row r sits at c ^ ((r >> 1) & 7), so the fragment
// reads (32 rows x one chunk per half-wave) hit distinct banks.  The MFMA is
// v_mfma_f32_32x32x16_bf16 with the vocabulary as its M side: a lane's 16
// accumulators are 16 vocabulary entries of one hidden row, so the row
// statistics are in-lane plus one exchange with lane ^ 32.
#include "kernels.hpp"
#include "stats.hpp"

namespace wedlm {

namespace {
constexpr int kNW = 8;                            // waves per work-group: 4 (vocab) x 2 (rows)
constexpr int kAhead = 2;                         // stages in flight beyond the one computed
constexpr int kSlots = kAhead + 1;
constexpr int kRowB = kLmKC * 2;                  // bytes of one row in a stage (128)
constexpr int kABytes = kLmNT * kRowB;            // weight rows of a stage (32 KB)
constexpr int kBBytes = kLmMT * kRowB;            // hidden rows of a stage (16 KB)
constexpr int kSlotB = kABytes + kBBytes;
constexpr int kLPS = kSlotB / 1024 / kNW;         // DMA instructions per wave per stage (6)
static_assert(kLPS * 1024 * kNW == kSlotB, "a stage must split into whole wave loads");
static_assert(kRowB == 128, "the chunk swizzle assumes 8 chunks per row");

__device__ __forceinline__ int lm_swz(int row, int c) { return c ^ ((row >> 1) & 7); }

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

__global__ __launch_bounds__(512) void lmhead_stats(LmheadArgs a) {
    __shared__ __attribute__((aligned(1024))) char s_ring[kSlots * kSlotB];
    __shared__ int s_rows[kLmMT];
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
    const int c0 = rg * kLmMT;
    if (c0 >= cnt) return;
    if (tid < kLmMT) s_rows[tid] = a.rows[min(c0 + tid, cnt - 1)];   // rows past the count repeat a valid one
    __syncthreads();
    const int n0 = vt * kLmNT;
    const int ns = a.Dm / kLmKC;
    const size_t rowbytes = (size_t)a.Dm * 2;

    // DMA sources of this lane: instruction q of a stage loads 8 row slices
    // (weights for q < kLmNT/8, then hidden rows); the lane that fills LDS
    // chunk (row, lane & 7) reads global chunk lm_swz(row, lane & 7).
    const char* gsrc[kLPS];
    uint32_t ldst[kLPS];
#pragma unroll
    for (int u = 0; u < kLPS; ++u) {
        const int q = w * kLPS + u;
        if (q < kLmNT / 8) {
            const int row = q * 8 + (lane >> 3);
            const int n = min(n0 + row, a.V - 1);   // past the vocabulary: a valid row, masked below
            gsrc[u] = reinterpret_cast<const char*>(a.lm_head) + (size_t)n * rowbytes + lm_swz(row, lane & 7) * 16;
            ldst[u] = q * 1024;
        } else {
            const int m = (q - kLmNT / 8) * 8 + (lane >> 3);
            gsrc[u] = reinterpret_cast<const char*>(a.hidden) + (size_t)s_rows[m] * rowbytes + lm_swz(m, lane & 7) * 16;
            ldst[u] = kABytes + (q - kLmNT / 8) * 1024;
        }
    }
    auto issue = [&](int st) {
        char* slot = s_ring + (st % kSlots) * kSlotB;
#pragma unroll
        for (int u = 0; u < kLPS; ++u)
            __builtin_amdgcn_global_load_lds(
                (const void*)(gsrc[u] + (size_t)st * kRowB),
                (__attribute__((address_space(3))) void*)(reinterpret_cast<uintptr_t>(slot + ldst[u])), 16, 0, 0);
    };

    // wave (wn, wm): vocabulary rows wn*64 .. +64 (two 32-tiles) x hidden
    // rows wm*64 .. +64 (two 32-tiles)
    const int wn = w & 3, wm = w >> 2;
    const int hl = lane >> 5, col = lane & 31;
    uint32_t aoff[2], boff[2];
    int arow[2], brow[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        arow[t] = wn * 64 + t * 32 + col;
        brow[t] = wm * 64 + t * 32 + col;
        aoff[t] = arow[t] * kRowB;
        boff[t] = kABytes + brow[t] * kRowB;
    }
    f32x16 acc[2][2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[x][y][e] = 0.f;

    const int npro = ns < kAhead ? ns : kAhead;
    for (int st = 0; st < npro; ++st) issue(st);
    for (int st = 0; st < ns; ++st) {
        // this wave's loads of stage st have landed (later stages may still
        // be in flight); the barrier publishes every wave's part and frees
        // the slot of stage st-1 for stage st+kAhead
        if (st + 1 < ns) lm_wait_vm<kLPS * (kAhead - 1)>();
        else lm_wait_vm<0>();
        lm_block_sync();
        if (st + kAhead < ns) issue(st + kAhead);
        const char* slot = s_ring + (st % kSlots) * kSlotB;
#pragma unroll
        for (int s = 0; s < kLmKC / 16; ++s) {
            bf16x8 af[2], bf[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                af[t] = *reinterpret_cast<const bf16x8*>(slot + aoff[t] + lm_swz(arow[t], 2 * s + hl) * 16);
                bf[t] = *reinterpret_cast<const bf16x8*>(slot + boff[t] + lm_swz(brow[t], 2 * s + hl) * 16);
            }
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int y = 0; y < 2; ++y)
                    acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[x], bf[y], acc[x][y], 0, 0, 0);
        }
    }

    // ---- statistics of this tile per hidden row
    lm_block_sync();   // every wave is done with the ring
    float4* s_stat = reinterpret_cast<float4*>(s_ring);   // [4 vocab waves][kLmMT]
#pragma unroll
    for (int y = 0; y < 2; ++y) {
        // the lane's 32 values in increasing vocabulary order: tile x, then
        // accumulator e (entry (e / 4) * 8 + hl * 4 + e % 4 of the 32-tile)
        float z[32];
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int v = n0 + wn * 64 + x * 32 + (e >> 2) * 8 + hl * 4 + (e & 3);
                z[x * 16 + e] = v < a.V ? acc[x][y][e] : -INFINITY;
            }
        float bm = z[0];
#pragma unroll
        for (int k = 1; k < 32; ++k) bm = fmaxf(bm, z[k]);
        Stat st{-INFINITY, 0x7fffffff, 0.f, 0.f};
        if (bm > -INFINITY) {
            int ba = 0x7fffffff;
#pragma unroll
            for (int k = 31; k >= 0; --k)   // backwards, so the first match wins
                if (z[k] == bm) ba = n0 + wn * 64 + (k >> 4) * 32 + ((k & 15) >> 2) * 8 + hl * 4 + (k & 3);
            st.m = bm;
            st.a = ba;
        }
        float s = 0.f, t = 0.f;
#pragma unroll
        for (int k = 0; k < 32; ++k) add_term(s, t, z[k], st.m);
        st.s = s;
        st.t = t;
        st = merge(st, shfl_xor_stat(st, 32));
        if (hl == 0)
            s_stat[wn * kLmMT + wm * 64 + y * 32 + col] = make_float4(st.m, __int_as_float(st.a), st.s, st.t);
    }
    __syncthreads();
    if (tid < kLmMT && c0 + tid < cnt) {
        const float4 p0 = s_stat[tid];
        Stat o{p0.x, __float_as_int(p0.y), p0.z, p0.w};
#pragma unroll
        for (int k = 1; k < 4; ++k) {
            const float4 p = s_stat[k * kLmMT + tid];
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
    hipLaunchKernelGGL(lmhead_stats, dim3(8u * nvt8 * (unsigned)a.nrg), dim3(512), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lmhead_merge, dim3((unsigned)a.R), dim3(64), 0, st, a);
    return hipGetLastError();
}

}  // namespace wedlm
