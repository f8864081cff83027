// model.hip -- the layers around the decode-step path for a whole synthetic
// decoder: token embedding, RMSNorm, the window's projections (split-K GEMM
// on the tile contraction of mma_tile.hpp), residual adds and the SwiGLU
// MLP.  wedlm_model_step (api.hip) strings these together with the
// reorder / attention / LM-head + select kernels into one decode step.
//
// Pages: WeDLM paper-summary page, TL;DR (the backbone is Qwen3-8B, a
// decoder-only transformer) and "Method" (a decode step is a causal forward
// of the reordered window over the cached prefix, then commit / select /
// refill).  The layer itself is not on the pages; this library takes the
// plain pre-norm decoder block: h = RMSNorm(x); x += Wo Attn(Wq h, Wk h,
// Wv h); h = RMSNorm(x); x += Wd (silu(Wg h) * (Wu h)).
//
// Storage points: the residual stream x is fp32; normalised activations,
// projections, attention outputs and the MLP activation are bf16 (the
// GEMM operands).  A projection y = h W^T is computed as S split-K partial
// products in fp32 (one work-group per (output tile, row group, K split)),
// summed by the kernel that consumes it.  q, k and v are one launch over
// the three weight matrices stacked along the output dimension, and so are
// the gate and up projections of the MLP.
#include "kernels.hpp"
#include "mma_tile.hpp"

namespace wedlm {

// up to 128 rows: 256 output columns x all rows per work-group
using GemmSmall = TileCfg<256, 128, 64, 3, 4>;
// more rows (the pages' window of 64 over a few sequences): 128 output
// columns x 256 rows per work-group, so a projection of a few thousand
// outputs splits K at most 8 ways to fill the chip and the fp32 partials
// stay small next to the weights
using GemmRows = TileCfg<128, 256, 64, 3, 2>;
// the plain projections at more rows: 256 output columns x 128 rows per
// work-group, the row groups of one output tile on one XCD so the second
// reads the weight tile from that XCD's L2 (the SwiGLU form keeps the
// 256-row tile, whose epilogue pairs the gate and up columns)
using GemmWide = TileCfg<256, 128, 64, 3, 4>;

__device__ __forceinline__ float silu(float g) { return g / (1.f + __expf(-g)); }


// Row kernels run one work-group of kRowThreads threads per row: a thread
// owns the float4 columns tid, tid + kRowThreads, ... (one each at a
// 4096-wide row), so 16 waves per row keep the partial reads in flight.
constexpr int kRowThreads = 1024;

// Sum over the work-group (kRowThreads / 64 waves).
__device__ __forceinline__ float block_sum(float v, float* s_red) {
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = v;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kRowThreads / 64; ++w) t += s_red[w];
    return t;
}

// h[m] = RMSNorm(x_res[m]) * g (bf16), x_res[m] already final and written
// by this same thread for its own columns.
__device__ __forceinline__ void rmsnorm_row(const ModelRowArgs& a, int m, float ss, float* s_red) {
    const int N4 = a.N / 4;
    const float rs = rsqrtf(block_sum(ss, s_red) / a.N + a.eps);
    const float4* x = reinterpret_cast<const float4*>(a.x_res + (size_t)m * a.N);
    const uint2* g = reinterpret_cast<const uint2*>(a.g);
    uint2* h = reinterpret_cast<uint2*>(a.h + (size_t)m * a.N);
    for (int c = threadIdx.x; c < N4; c += kRowThreads) {
        const float4 v = x[c];
        const float4 w = unpack_bf16x4(g[c]);
        h[c] = pack_bf16x4(make_float4(v.x * rs * w.x, v.y * rs * w.y, v.z * rs * w.z, v.w * rs * w.w));
    }
}

// x_res[m] = E[tok[m]] (fp32); h[m] = RMSNorm(x_res[m]) * g (bf16).
__global__ __launch_bounds__(kRowThreads) void embed_rmsnorm(ModelRowArgs a) {
    const int m = blockIdx.x;
    __shared__ float s_red[kRowThreads / 64];
    int t = a.tok[m];
    if (t < 0 || t >= a.n_embed) {
        if (threadIdx.x == 0) set_status(a.status, WEDLM_DEV_BAD_TOKEN);
        t = 0;
    }
    const int N4 = a.N / 4;
    const uint2* e = reinterpret_cast<const uint2*>(a.embed + (size_t)t * a.N);
    float4* x = reinterpret_cast<float4*>(a.x_res + (size_t)m * a.N);
    float ss = 0.f;
    for (int c = threadIdx.x; c < N4; c += kRowThreads) {
        const float4 v = unpack_bf16x4(e[c]);
        x[c] = v;
        ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    rmsnorm_row(a, m, ss, s_red);
}

// x_res[m] += sum_s P[s][m] (in split order); h[m] = RMSNorm(x_res[m]) * g.
__global__ __launch_bounds__(kRowThreads) void add_rmsnorm(ModelRowArgs a) {
    const int m = blockIdx.x;
    __shared__ float s_red[kRowThreads / 64];
    const int N4 = a.N / 4;
    float4* x = reinterpret_cast<float4*>(a.x_res + (size_t)m * a.N);
    const float4* P = reinterpret_cast<const float4*>(a.P) + (size_t)m * N4;
    const size_t plane4 = (size_t)a.M * N4;
    float ss = 0.f;
    for (int c = threadIdx.x; c < N4; c += kRowThreads) {
        float4 v = x[c];
        for (int s = 0; s < a.S; ++s) v = add4(v, P[s * plane4 + c]);
        x[c] = v;
        ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    rmsnorm_row(a, m, ss, s_red);   // re-reads only this thread's own columns
}

// Sum of the S partials of four consecutive columns (4c .. 4c+3) of row m.
__device__ __forceinline__ float4 sum_splits(const ModelRowArgs& a, size_t i4) {
    const float4* P = reinterpret_cast<const float4*>(a.P);
    const size_t plane4 = (size_t)a.M * a.N / 4;
    float4 v = P[i4];
    for (int s = 1; s < a.S; ++s) v = add4(v, P[s * plane4 + i4]);
    return v;
}

// SwiGLU activation from the stacked gate / up projection (N = 2F columns,
// gate first): h[m][n] = bf16(silu(gate[m][n]) * up[m][n]), n < F.
__global__ __launch_bounds__(256) void finish_swiglu(ModelRowArgs a) {
    const int F4 = a.N / 8;
    const size_t total4 = (size_t)a.M * F4;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < total4; i += (size_t)gridDim.x * 256) {
        const int m = (int)(i / F4);
        const int c = (int)(i - (size_t)m * F4);
        const size_t row4 = (size_t)m * (2 * F4);
        const float4 g = sum_splits(a, row4 + c);
        const float4 u = sum_splits(a, row4 + F4 + c);
        reinterpret_cast<uint2*>(a.h)[i] =
            pack_bf16x4(make_float4(silu(g.x) * u.x, silu(g.y) * u.y, silu(g.z) * u.z, silu(g.w) * u.w));
    }
}

// Gate and up rows interleaved by tiles of 128: rows [0, 64) of tile t are
// gate rows 64t .. 64t+63, rows [64, 128) the up rows of the same outputs,
// so one work-group holds both factors of every SwiGLU output it owns.
struct PairedRows {
    const char* gate;
    const char* up;
    size_t rowbytes;
    __device__ const char* operator()(int n) const {
        // arithmetic choice of the base (a conditional between the two
        // members would become a dynamically indexed field load and keep
        // the functor in memory)
        const int r = n & 127;
        const uintptr_t g = reinterpret_cast<uintptr_t>(gate), u = reinterpret_cast<uintptr_t>(up);
        const uintptr_t base = g + (uintptr_t)(r >> 6) * (u - g);
        return reinterpret_cast<const char*>(base) + (size_t)((n >> 7) * 64 + (r & 63)) * rowbytes;
    }
};

// The SwiGLU epilogue of one 128 x 256 tile (WN = 2): the waves holding the
// up rows (wave_n 1) pass their accumulators through LDS to the waves
// holding the gate rows of the same outputs (wave_n 0), which write
// act[m][c] = bf16(silu(g) * u) -- a lane's 16 values of one 32-row block
// are 4 runs of 4 consecutive outputs.
template <class C>
__device__ __forceinline__ void swiglu_epilogue(const GemmArgs& a, int m0, int tile, char* s_ring,
                                                const f32x16 (&acc)[C::TN][C::TM]) {
    static_assert(C::NT == 128 && C::WN == 2 && C::TN == 2, "paired tile shape");
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wn = C::wave_n(), wm = C::wave_m();
    const int hl = lane >> 5, col = lane & 31;
    float* s_up = reinterpret_cast<float*>(s_ring);    // [wm][x][y][e][lane]
    tile_block_sync();                                   // every wave is done with the ring
    if (wn == 1) {
#pragma unroll
        for (int x = 0; x < C::TN; ++x)
#pragma unroll
            for (int y = 0; y < C::TM; ++y)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    s_up[(((wm * C::TN + x) * C::TM + y) * 16 + e) * 64 + lane] = acc[x][y][e];
    }
    __syncthreads();
    if (wn != 0) return;
    const int F = a.N / 2;
#pragma unroll
    for (int y = 0; y < C::TM; ++y) {
        const int m = m0 + (wm * C::TM + y) * 32 + col;
        if (m >= a.M) continue;
#pragma unroll
        for (int x = 0; x < C::TN; ++x)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int c = tile * 64 + x * 32 + g4 * 8 + hl * 4;
                float v[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int e = 4 * g4 + i;
                    const float u = s_up[(((wm * C::TN + x) * C::TM + y) * 16 + e) * 64 + lane];
                    v[i] = silu(acc[x][y][e]) * u;
                }
                if (c < F)
                    *reinterpret_cast<uint2*>(a.act + (size_t)m * F + c) = pack_bf16x4(make_float4(v[0], v[1], v[2], v[3]));
            }
    }
}

// P[s][m][n] = sum over the s-th K range of X[m][k] W[n][k], fp32, W the
// stacked weight rows (or, in the SwiGLU form, the activation directly).  Work-group i: split s = i % S (so the work-groups of
// one K range share an XCD when S divides 8 or 8 divides S), then row
// group, then output tile.  On the 128-row tile with several row groups
// the ids of one (output tile, split) unit's row groups lie 8 apart
// (consecutive ids go round the 8 XCDs), so they share an XCD and its L2:
// i = (u / 8 * nrg + mg) * 8 + u % 8 for unit u = nt * S + s, the grid
// padded to whole groups of 8 units.
template <class C>
__global__ __launch_bounds__(64 * C::NW) void gemm_split(GemmArgs a) {
    __shared__ __attribute__((aligned(1024))) char s_ring[C::SLOTS * C::SLOTB];
    __shared__ int s_rows[C::MT];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int i = blockIdx.x;
    int s, mg, nt;
    if (C::MT == 128 && a.nrg > 1) {
        const int j = i >> 3;
        mg = j % a.nrg;
        const int u = (j / a.nrg) * 8 + (i & 7);
        s = u % a.S;
        nt = u / a.S;
        if (nt * C::NT >= a.N) return;  // padding: the whole work-group leaves
    } else {
        s = i % a.S;
        mg = (i / a.S) % a.nrg;
        nt = i / a.S / a.nrg;
    }
    const int m0 = mg * C::MT, n0 = nt * C::NT;
    if (tid < C::MT) s_rows[tid] = min(m0 + tid, a.M - 1);
    __syncthreads();
    const int kr = a.K / a.S;
    const size_t k0b = (size_t)s * kr * 2;
    f32x16 acc[C::TN][C::TM];
    if constexpr (C::NT == 128 && C::WN == 2 && C::TN == 2) {
        if (a.act) {
            const PairedRows rows{reinterpret_cast<const char*>(a.W0), reinterpret_cast<const char*>(a.W1),
                                  (size_t)a.K * 2};
            tile_mma_rows<C>(rows, n0, a.N, reinterpret_cast<const char*>(a.X), s_rows, a.K, a.K, s_ring, acc,
                             a.M - m0);
            swiglu_epilogue<C>(a, m0, nt, s_ring, acc);
            return;
        }
    }
    const StackedRows rows{reinterpret_cast<const char*>(a.W0) + k0b, reinterpret_cast<const char*>(a.W1) + k0b,
                           reinterpret_cast<const char*>(a.W2) + k0b, a.n1, a.n2, (size_t)a.K * 2};
    tile_mma_rows<C>(rows, n0, a.N, reinterpret_cast<const char*>(a.X) + k0b, s_rows, kr, a.K, s_ring, acc, a.M - m0);
    const int wn = C::wave_n(), wm = C::wave_m();
    const int hl = lane >> 5, col = lane & 31;
    float* P = a.P + (size_t)s * a.M * a.N;
#pragma unroll
    for (int y = 0; y < C::TM; ++y) {
        const int m = m0 + (wm * C::TM + y) * 32 + col;
        if (m >= a.M) continue;
#pragma unroll
        for (int x = 0; x < C::TN; ++x)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int n = n0 + (wn * C::TN + x) * 32 + g4 * 8 + hl * 4;
                if (n < a.N)
                    *reinterpret_cast<float4*>(P + (size_t)m * a.N + n) =
                        make_float4(acc[x][y][4 * g4], acc[x][y][4 * g4 + 1], acc[x][y][4 * g4 + 2],
                                    acc[x][y][4 * g4 + 3]);
            }
    }
}

// Split count of one projection: the largest power of two (at most 16)
// that keeps the launch within one work-group per CU (256) -- or, for
// the small tile, the smallest that reaches it -- with K ranges that are
// whole stages and at least four of them.
int gemm_splits(int M, int N, int K) {
    const bool small = M <= GemmSmall::MT;
    const int nt = small ? (N + GemmSmall::NT - 1) / GemmSmall::NT : (N + GemmRows::NT - 1) / GemmRows::NT;
    const int mt = small ? 1 : (M + GemmRows::MT - 1) / GemmRows::MT;
    const int kc = small ? GemmSmall::KC : GemmRows::KC;
    int S = 1;
    auto can_double = [&](int s) { return s < 16 && K % (2 * s * kc) == 0 && K / (2 * s) >= 4 * kc; };
    if (small) {
        while (nt * mt * S < 256 && can_double(S)) S *= 2;
    } else {
        while (nt * mt * 2 * S <= 256 && can_double(S)) S *= 2;
    }
    return S;
}

// The SwiGLU form runs on the 256-row tile with a single K split.
bool gemm_swiglu_fused(int M, int S) { return M > GemmSmall::MT && S == 1; }

hipError_t launch_gemm(GemmArgs a, hipStream_t st) {
    if (a.act && !gemm_swiglu_fused(a.M, a.S)) return hipErrorInvalidValue;
    if (a.M <= GemmSmall::MT) {
        a.nrg = 1;
        const unsigned g = (unsigned)(((a.N + GemmSmall::NT - 1) / GemmSmall::NT) * a.S);
        hipLaunchKernelGGL(gemm_split<GemmSmall>, dim3(g), dim3(64 * GemmSmall::NW), 0, st, a);
    } else if (!a.act) {
        a.nrg = (a.M + GemmWide::MT - 1) / GemmWide::MT;
        const unsigned units = (unsigned)(((a.N + GemmWide::NT - 1) / GemmWide::NT) * a.S);
        const unsigned g = (units + 7) / 8 * 8 * (unsigned)a.nrg;
        hipLaunchKernelGGL(gemm_split<GemmWide>, dim3(g), dim3(64 * GemmWide::NW), 0, st, a);
    } else {
        a.nrg = (a.M + GemmRows::MT - 1) / GemmRows::MT;
        const unsigned g = (unsigned)(((a.N + GemmRows::NT - 1) / GemmRows::NT) * a.nrg * a.S);
        hipLaunchKernelGGL(gemm_split<GemmRows>, dim3(g), dim3(64 * GemmRows::NW), 0, st, a);
    }
    return hipGetLastError();
}

hipError_t launch_embed_rmsnorm(const ModelRowArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(embed_rmsnorm, dim3((unsigned)a.M), dim3(kRowThreads), 0, st, a);
    return hipGetLastError();
}
hipError_t launch_add_rmsnorm(const ModelRowArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(add_rmsnorm, dim3((unsigned)a.M), dim3(kRowThreads), 0, st, a);
    return hipGetLastError();
}
static unsigned row_blocks(size_t items) {
    const size_t b = (items + 255) / 256;
    return (unsigned)(b < 4096 ? b : 4096);
}
hipError_t launch_finish_swiglu(const ModelRowArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(finish_swiglu, dim3(row_blocks((size_t)a.M * a.N / 8)), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace wedlm
