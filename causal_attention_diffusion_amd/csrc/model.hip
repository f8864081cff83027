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
// products in fp32 (one work-group per (256-wide output tile, row group,
// K split)), summed by the kernel that consumes it.
#include "kernels.hpp"
#include "mma_tile.hpp"

namespace wedlm {

using GemmSmall = TileCfg<256, 128, 64, 3, 4>;   // up to 128 rows
using GemmLarge = TileCfg<256, 256, 32, 4, 2>;   // 129 .. 256 rows per row group

__device__ __forceinline__ float silu(float g) { return g / (1.f + __expf(-g)); }

// x_res[m] = E[tok[m]] (fp32); h[m] = RMSNorm(x_res[m]) * g (bf16).
// One work-group per row.
__global__ __launch_bounds__(256) void embed_rmsnorm(ModelRowArgs a) {
    const int m = blockIdx.x;
    __shared__ float s_red[4];
    int t = a.tok[m];
    if (t < 0 || t >= a.n_embed) {
        if (threadIdx.x == 0) set_status(a.status, WEDLM_DEV_BAD_TOKEN);
        t = 0;
    }
    const bf16_t* e = a.embed + (size_t)t * a.N;
    float* x = a.x_res + (size_t)m * a.N;
    float ss = 0.f;
    for (int n = threadIdx.x; n < a.N; n += 256) {
        const float v = bf16_to_f32(e[n].bits);
        x[n] = v;
        ss += v * v;
    }
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float rs = rsqrtf((s_red[0] + s_red[1] + s_red[2] + s_red[3]) / a.N + a.eps);
    bf16_t* h = a.h + (size_t)m * a.N;
    for (int n = threadIdx.x; n < a.N; n += 256)
        h[n].bits = f32_to_bf16(x[n] * rs * bf16_to_f32(a.g[n].bits));
}

// x_res[m] += sum_s P[s][m]; h[m] = RMSNorm(x_res[m]) * g (bf16).
__global__ __launch_bounds__(256) void add_rmsnorm(ModelRowArgs a) {
    const int m = blockIdx.x;
    __shared__ float s_red[4];
    float* x = a.x_res + (size_t)m * a.N;
    const size_t plane = (size_t)a.M * a.N;
    float ss = 0.f;
    for (int n = threadIdx.x; n < a.N; n += 256) {
        float v = x[n];
        for (int s = 0; s < a.S; ++s) v += a.P[s * plane + (size_t)m * a.N + n];
        x[n] = v;
        ss += v * v;
    }
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float rs = rsqrtf((s_red[0] + s_red[1] + s_red[2] + s_red[3]) / a.N + a.eps);
    bf16_t* h = a.h + (size_t)m * a.N;
    for (int n = threadIdx.x; n < a.N; n += 256)
        h[n].bits = f32_to_bf16(x[n] * rs * bf16_to_f32(a.g[n].bits));
}

// out[m][n] = bf16(sum_s P[s][m][n]) (gate == nullptr), or
// out[m][n] = bf16(silu(sum_s Pg) * sum_s P) with Pg = gate partials.
__global__ __launch_bounds__(256) void finish_rows(ModelRowArgs a) {
    const size_t total = (size_t)a.M * a.N;
    const size_t plane = total;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (size_t)gridDim.x * 256) {
        float v = 0.f;
        for (int s = 0; s < a.S; ++s) v += a.P[s * plane + i];
        if (a.Pg) {
            float g = 0.f;
            for (int s = 0; s < a.S; ++s) g += a.Pg[s * plane + i];
            v *= silu(g);
        }
        a.h[i].bits = f32_to_bf16(v);
    }
}

// P[s][m][n] = sum over the s-th K range of X[m][k] W[n][k], fp32.
// Work-group i: split s = i % S, then row group, then output tile.
template <class C>
__global__ __launch_bounds__(64 * C::NW) void gemm_split(GemmArgs a) {
    __shared__ __attribute__((aligned(1024))) char s_ring[C::SLOTS * C::SLOTB];
    __shared__ int s_rows[C::MT];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int i = blockIdx.x;
    const int s = i % a.S;
    const int mg = (i / a.S) % a.nrg;
    const int nt = i / a.S / a.nrg;
    const int m0 = mg * C::MT, n0 = nt * C::NT;
    if (tid < C::MT) s_rows[tid] = min(m0 + tid, a.M - 1);
    __syncthreads();
    const int kr = a.K / a.S;
    const size_t k0b = (size_t)s * kr * 2;
    f32x16 acc[C::TN][C::TM];
    tile_mma<C>(reinterpret_cast<const char*>(a.W) + k0b, n0, a.N, reinterpret_cast<const char*>(a.X) + k0b, s_rows,
                kr, a.K, s_ring, acc);
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

// Split count and launch of one projection.
int gemm_splits(int M, int N, int K) {
    const int nt = (N + 255) / 256;
    const int mt = M <= GemmSmall::MT ? 1 : (M + GemmLarge::MT - 1) / GemmLarge::MT;
    const int kc = M <= GemmSmall::MT ? GemmSmall::KC : GemmLarge::KC;
    int S = 1;
    while (nt * mt * S < 256 && S < 16 && K % (2 * S * kc) == 0 && K / (2 * S) >= 4 * kc) S *= 2;
    return S;
}

hipError_t launch_gemm(GemmArgs a, hipStream_t st) {
    if (a.M <= GemmSmall::MT) {
        a.nrg = 1;
        const unsigned g = (unsigned)(((a.N + GemmSmall::NT - 1) / GemmSmall::NT) * a.S);
        hipLaunchKernelGGL(gemm_split<GemmSmall>, dim3(g), dim3(64 * GemmSmall::NW), 0, st, a);
    } else {
        a.nrg = (a.M + GemmLarge::MT - 1) / GemmLarge::MT;
        const unsigned g = (unsigned)(((a.N + GemmLarge::NT - 1) / GemmLarge::NT) * a.nrg * a.S);
        hipLaunchKernelGGL(gemm_split<GemmLarge>, dim3(g), dim3(64 * GemmLarge::NW), 0, st, a);
    }
    return hipGetLastError();
}

hipError_t launch_embed_rmsnorm(const ModelRowArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(embed_rmsnorm, dim3((unsigned)a.M), dim3(256), 0, st, a);
    return hipGetLastError();
}
hipError_t launch_add_rmsnorm(const ModelRowArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(add_rmsnorm, dim3((unsigned)a.M), dim3(256), 0, st, a);
    return hipGetLastError();
}
hipError_t launch_finish_rows(const ModelRowArgs& a, hipStream_t st) {
    const size_t total = (size_t)a.M * a.N;
    const size_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(finish_rows, dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace wedlm
