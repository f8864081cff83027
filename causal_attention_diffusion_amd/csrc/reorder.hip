// reorder.hip -- Topological Reordering, RoPE at logical positions and KV
// append for one WeDLM decode step.
//
// Pages: "WeDLM: Reconciling Diffusion Language Models with Standard Causal
// Attention for Fast Inference", paper-summary page, "Key claims" (paper
// sec. 4.1, Eq. 5-6: observed tokens go to the physical front, RoPE keeps
// their logical positions) and "Method" (inference paragraph: the window is
// reordered with filled tokens first before the causal pass on the cache).
//
// One work-group per (physical row r, sequence b).  Each wave derives the
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
    const int lane = tid & 63;

    // Every wave derives the permutation entry of row r by itself: no LDS,
    // no barrier, and the loads below overlap.
    const bool in = lane < W;
    const int f = in ? a.filled[(size_t)b * W + lane] : 0;
    const int p_lane = in ? a.pos[(size_t)b * W + lane] : 0;
    const int L = a.ctx_len[b];
    const uint64_t fm = __ballot(in && f != 0);
    const uint64_t mm = __ballot(in && f == 0);
    const uint64_t below = lane == 0 ? 0ull : ((1ull << lane) - 1ull);
    const int n_obs = __popcll(fm);
    const int phys = f ? __popcll(fm & below) : n_obs + __popcll(mm & below);
    const uint64_t hit = __ballot(in && phys == r);
    const int slot = (int)__builtin_ctzll(hit);   // the map slot -> phys is a bijection onto [0, W)
    const int p = __shfl(p_lane, slot);

    const bool ctx_ok = L >= 0 && (int64_t)L + W <= (int64_t)a.max_pages * kPage;
    int page = -1;
    if (ctx_ok) {
        page = a.block_table[(size_t)b * a.max_pages + (L + r) / kPage];
        if (page < 0 || page >= a.num_pages) page = -1;
    }
    if (tid == 0) {
        a.perm[(size_t)b * W + r] = slot;
        if (!ctx_ok) set_status(a.status, WEDLM_DEV_BAD_CTX);
        else if (page < 0) set_status(a.status, WEDLM_DEV_BAD_PAGE);
    }
    if (tid < 64 && r == 0) {
        const int p_prev = __shfl_up(p_lane, 1);
        const bool bad_pos = in && (p_lane < 0 || (lane > 0 && p_lane <= p_prev));
        if (__ballot(bad_pos) && lane == 0) set_status(a.status, WEDLM_DEV_BAD_POS);
    }

    // cos/sin of the D/2 pair angles, float64, once per work-group
    __shared__ double s_cs[64], s_sn[64];
    if (tid < half) {
        double sn, cs;
        sincos((double)p * exp2(-(2.0 * tid / D) * a.log2_base), &sn, &cs);
        s_cs[tid] = cs;
        s_sn[tid] = sn;
    }
    __syncthreads();

    // Work items are 4 consecutive pairs (c .. c+3 with c+D/2 .. c+D/2+3) of
    // one head: Hq query heads, then Hkv key heads; value rows are copied in
    // 4-element pieces.  Each thread loads all of its items before it
    // computes, so the loads overlap.
    constexpr int kMaxItems = 4;
    const int qn = a.Hq * (half / 4), kn = a.Hkv * (half / 4), vn = a.Hkv * (D / 4);
    const int t_row = L + r;
    const size_t row0 = page >= 0 ? ((size_t)page * a.Hkv) * kPage + (t_row % kPage) : 0;
    const T* qs = static_cast<const T*>(a.q) + ((size_t)b * W + slot) * a.Hq * D;
    T* qd = static_cast<T*>(a.q_phys) + ((size_t)b * W + r) * a.Hq * D;
    const T* ks = static_cast<const T*>(a.k) + ((size_t)b * W + slot) * a.Hkv * D;
    const T* vs = static_cast<const T*>(a.v) + ((size_t)b * W + slot) * a.Hkv * D;
    T* kc = static_cast<T*>(a.k_cache);
    T* vc = static_cast<T*>(a.v_cache);
    const int n_items = qn + (page >= 0 ? kn + vn : 0);
    for (int base = tid; base < n_items; base += kMaxItems * 256) {
        float x0[kMaxItems][4], x1[kMaxItems][4];
#pragma unroll
        for (int u = 0; u < kMaxItems; ++u) {
            const int it = base + u * 256;
            if (it >= n_items) continue;
            if (it < qn + kn) {
                const bool isq = it < qn;
                const int j = isq ? it : it - qn;
                const int hh = j / (half / 4), c = (j % (half / 4)) * 4;
                const T* src = (isq ? qs : ks) + (size_t)hh * D + c;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    x0[u][e] = DT<T>::load(src, e);
                    x1[u][e] = DT<T>::load(src, e + half);
                }
            } else {
                const int j = it - qn - kn;
                const T* src = vs + (size_t)j * 4;
#pragma unroll
                for (int e = 0; e < 4; ++e) x0[u][e] = DT<T>::load(src, e);
            }
        }
#pragma unroll
        for (int u = 0; u < kMaxItems; ++u) {
            const int it = base + u * 256;
            if (it >= n_items) continue;
            if (it < qn + kn) {
                const bool isq = it < qn;
                const int j = isq ? it : it - qn;
                const int hh = j / (half / 4), c = (j % (half / 4)) * 4;
                T* dst = isq ? qd + (size_t)hh * D + c : kc + (row0 + (size_t)hh * kPage) * D + c;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const double cs = s_cs[c + e], sn = s_sn[c + e];
                    const double y0 = (double)x0[u][e] * cs - (double)x1[u][e] * sn;
                    const double y1 = (double)x1[u][e] * cs + (double)x0[u][e] * sn;
                    DT<T>::store(dst, e, (float)y0);
                    DT<T>::store(dst, e + half, (float)y1);
                }
            } else {
                const int j = it - qn - kn;
                const int g = j / (D / 4), d = (j % (D / 4)) * 4;
                T* dst = vc + (row0 + (size_t)g * kPage) * D + d;
#pragma unroll
                for (int e = 0; e < 4; ++e) DT<T>::store(dst, e, x0[u][e]);
            }
        }
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
