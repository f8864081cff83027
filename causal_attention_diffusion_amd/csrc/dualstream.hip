// dualstream.hip -- Dual-Stream Masking attention as a forward pass, built
// from the decode step's own kernels.
//
// Pages: WeDLM paper-summary page, "Method" (training paragraph) and "Key
// claims" (sec. 4.2, Eq. 8-10): a clean memory stream and a block-masked
// prediction stream share position ids; a prediction token of block i
// attends to the memory tokens whose logical positions precede block i.
// Inside its block it follows Topological Reordering under the causal mask
// (sec. 3.2, 4.1), and the memory stream is plainly causal (this library's
// reading where the page is silent).
//
// Every prediction block is then exactly a decode step: its window is the
// block (reordered by its flags) and its cached prefix is the memory
// stream's first i*b tokens.  The memory stream itself is a run of decode
// steps over all-observed 64-token windows.  So the whole pass is two
// (reorder, attention) pairs over one paged cache in the workspace:
//   memory:     S*N/64 windows; window c of sequence s sits at tokens
//               64c .. 64c+63 of the sequence's memory pages;
//   prediction: S*N/b windows; window i sees the memory pages of tokens
//               0 .. i*b-1 and writes its own K/V into private pages.
// dual_stream_layout fills the block tables, positions and prefix lengths.
#include "kernels.hpp"

namespace wedlm {

struct DualLayoutArgs {
    uint8_t* filled_m;   // [S*N] all 1 (memory windows are fully observed)
    int32_t* pos_m;      // [S*N]
    int32_t* ctx_m;      // [S*N/64]
    int32_t* bt_m;       // [S*N/64][N/16]
    int32_t* pos_p;      // [S*N]
    int32_t* ctx_p;      // [S*N/b]
    int32_t* bt_p;       // [S*N/b][N/16]
    int S, N, b;
};

// One thread per (window, page slot) of either call, plus the per-token
// arrays.  Memory page p of sequence s is s*N/16 + p; prediction page p is
// S*N/16 + s*N/16 + p.
__global__ __launch_bounds__(256) void dual_stream_layout(DualLayoutArgs a) {
    const int np = a.N / kPage;
    const long nm = (long)a.S * (a.N / 64), npred = (long)a.S * (a.N / a.b);
    const long total = (nm + npred) * np + (long)a.S * a.N;
    for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (long)gridDim.x * blockDim.x) {
        if (i < nm * np) {
            const long w = i / np;
            const int p = (int)(i - w * np);
            const int s = (int)(w / (a.N / 64));
            a.bt_m[i] = s * np + p;
            if (p == 0) a.ctx_m[w] = (int)(w - (long)s * (a.N / 64)) * 64;
        } else if (i < (nm + npred) * np) {
            const long k = i - nm * np;
            const long w = k / np;
            const int p = (int)(k - w * np);
            const int s = (int)(w / (a.N / a.b));
            const int start = (int)(w - (long)s * (a.N / a.b)) * a.b;
            a.bt_p[k] = p < start / kPage ? s * np + p : a.S * np + s * np + p;
            if (p == 0) a.ctx_p[w] = start;
        } else {
            const long t = i - (nm + npred) * np;
            const int n = (int)(t % a.N);
            a.filled_m[t] = 1;
            a.pos_m[t] = n;
            a.pos_p[t] = n;
        }
    }
}

hipError_t launch_dual_layout(uint8_t* filled_m, int32_t* pos_m, int32_t* ctx_m, int32_t* bt_m, int32_t* pos_p,
                              int32_t* ctx_p, int32_t* bt_p, int S, int N, int b, hipStream_t st) {
    DualLayoutArgs a{filled_m, pos_m, ctx_m, bt_m, pos_p, ctx_p, bt_p, S, N, b};
    const long total = ((long)S * (N / 64) + (long)S * (N / b)) * (N / kPage) + (long)S * N;
    const long blocks = (total + 255) / 256;
    hipLaunchKernelGGL(dual_stream_layout, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace wedlm
