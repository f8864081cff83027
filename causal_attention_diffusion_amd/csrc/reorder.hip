// reorder.hip -- Topological Reordering, RoPE at logical positions and KV
// append for one WeDLM decode step.
//
// Pages: "WeDLM: Reconciling Diffusion Language Models with Standard Causal
// Attention for Fast Inference", paper-summary page, "Key claims" (paper
// sec. 4.1, Eq. 5-6: observed tokens go to the physical front, RoPE keeps
// their logical positions) and "Method" (inference paragraph: the window is
// reordered with filled tokens first before the causal pass on the cache).
//
// One work-group per (physical row r, sequence b).  Wave 0 derives the
// permutation with two ballots (filled / masked masks) and a prefix
// popcount: slot i lands at physical row popc(filled below i) if filled,
// else n_obs + popc(masked below i).  The work-group then rotates the Hq
// query heads and Hkv key heads of that slot at its logical position and
// writes the key/value rows into the paged cache at token ctx_len[b] + r.
// The work is tiny (B*W*(Hq+2Hkv)*D elements) and latency-bound; angles and
// rotations are float64 so that positions up to 2^31 keep full accuracy.
#include "kernels.hpp"

namespace wedlm {


template <typename T>
__global__ __launch_bounds__(256) void reorder_rope_append(ReorderArgs a) {
    const int r = blockIdx.x;
    const int b = blockIdx.y;
    const int W = a.W, D = a.D, half = D / 2;
    const int tid = threadIdx.x;

    __shared__ int s_slot;
    __shared__ int s_page;  // -1: do not append (bad ctx_len or page)
    __shared__ int s_pos;
    __shared__ double s_cos[64], s_sin[64];

    if (tid < kWave) {
        const int lane = tid;
        const bool in = lane < W;
        const int f = in ? a.filled[(size_t)b * W + lane] : 0;
        const uint64_t fm = __ballot(in && f != 0);
        const uint64_t mm = __ballot(in && f == 0);
        const uint64_t below = lane == 0 ? 0ull : ((1ull << lane) - 1ull);
        const int n_obs = __popcll(fm);
        const int phys = f ? __popcll(fm & below) : n_obs + __popcll(mm & below);
        if (in && phys == r) s_slot = lane;
        const int p = in ? a.pos[(size_t)b * W + lane] : 0;
        const int p_prev = __shfl_up(p, 1);
        const bool bad_pos = in && (p < 0 || (lane > 0 && p <= p_prev));
        const uint64_t any_bad = __ballot(bad_pos);
        if (lane == 0) {
            if (any_bad && r == 0) set_status(a.status, WEDLM_DEV_BAD_POS);
            const int L = a.ctx_len[b];
            int page = -1;
            if (L < 0 || (int64_t)L + W > (int64_t)a.max_pages * kPage) {
                if (r == 0) set_status(a.status, WEDLM_DEV_BAD_CTX);
            } else {
                const int t = L + r;
                page = a.block_table[(size_t)b * a.max_pages + t / kPage];
                if (page < 0 || page >= a.num_pages) {
                    set_status(a.status, WEDLM_DEV_BAD_PAGE);
                    page = -1;
                }
            }
            s_page = page;
        }
    }
    __syncthreads();
    const int slot = s_slot;
    if (tid == 0) {
        a.perm[(size_t)b * W + r] = slot;
        s_pos = a.pos[(size_t)b * W + slot];
    }
    __syncthreads();
    const double p = (double)s_pos;
    if (tid < half) {
        const double inv_freq = exp2(-(2.0 * tid / D) * a.log2_base);
        double sn, cs;
        sincos(p * inv_freq, &sn, &cs);
        s_sin[tid] = sn;
        s_cos[tid] = cs;
    }
    __syncthreads();

    // queries: rotate and write in physical order
    const T* qs = static_cast<const T*>(a.q) + ((size_t)b * W + slot) * a.Hq * D;
    T* qd = static_cast<T*>(a.q_phys) + ((size_t)b * W + r) * a.Hq * D;
    for (int idx = tid; idx < a.Hq * half; idx += blockDim.x) {
        const int h = idx / half, c = idx - h * half;
        const double x0 = DT<T>::load(qs, h * D + c), x1 = DT<T>::load(qs, h * D + c + half);
        const double cs = s_cos[c], sn = s_sin[c];
        DT<T>::store(qd, h * D + c, (float)(x0 * cs - x1 * sn));
        DT<T>::store(qd, h * D + c + half, (float)(x1 * cs + x0 * sn));
    }

    const int page = s_page;
    if (page < 0) return;
    const int t = a.ctx_len[b] + r;
    const size_t row0 = ((size_t)page * a.Hkv) * kPage + (t % kPage);  // + g * kPage
    const T* ks = static_cast<const T*>(a.k) + ((size_t)b * W + slot) * a.Hkv * D;
    const T* vs = static_cast<const T*>(a.v) + ((size_t)b * W + slot) * a.Hkv * D;
    T* kc = static_cast<T*>(a.k_cache);
    T* vc = static_cast<T*>(a.v_cache);
    for (int idx = tid; idx < a.Hkv * half; idx += blockDim.x) {
        const int g = idx / half, c = idx - g * half;
        const double x0 = DT<T>::load(ks, g * D + c), x1 = DT<T>::load(ks, g * D + c + half);
        const double cs = s_cos[c], sn = s_sin[c];
        const size_t o = (row0 + (size_t)g * kPage) * D;
        DT<T>::store(kc, o + c, (float)(x0 * cs - x1 * sn));
        DT<T>::store(kc, o + c + half, (float)(x1 * cs + x0 * sn));
    }
    for (int idx = tid; idx < a.Hkv * D; idx += blockDim.x) {
        const int g = idx / D, d = idx - g * D;
        vc[(row0 + (size_t)g * kPage) * D + d] = vs[(size_t)g * D + d];
    }
}

hipError_t launch_reorder(const ReorderArgs& a, int dtype, hipStream_t stream) {
    dim3 grid(a.W, a.B), block(256);
    if (dtype == WEDLM_F32)
        hipLaunchKernelGGL(reorder_rope_append<float>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(reorder_rope_append<bf16_t>, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace wedlm
