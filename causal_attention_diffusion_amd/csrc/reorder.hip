// reorder.hip -- Topological Reordering, RoPE at logical positions and KV
// append for one WeDLM decode step.
//
// Pages: "WeDLM: Reconciling Diffusion Language Models with Standard Causal
// Attention for Fast Inference", paper-summary page, "Key claims" (paper
// sec. 4.1, Eq. 5-6: observed tokens go to the physical front, RoPE keeps
// their logical positions) and "Method" (inference paragraph: the window is
// reordered with filled tokens first before the causal pass on the cache).
//
// One work-group per (logical slot i, sequence b).  It loads the rows of
// slot i at once, and meanwhile each wave derives the slot's physical row
// with two ballots (filled / masked masks) and a prefix popcount: slot i
// lands at r = popc(filled below i) if filled, else n_obs + popc(masked
// below i).  The work-group then rotates the Hq query heads and Hkv key
// heads at the slot's logical position into physical row r and writes the
// key/value rows into the paged cache at token ctx_len[b] + r.
// The work is tiny (B*W*(Hq+2Hkv)*D elements) and latency-bound; angles and
// rotations are float64 so that positions up to 2^31 keep full accuracy.
#include "kernels.hpp"

namespace wedlm {


// 4 consecutive elements (8-byte bf16 / 16-byte fp32 access; the offsets
// used here are multiples of 4 elements, so the accesses are aligned)
__device__ __forceinline__ void load4(const float* p, float (&x)[4]) {
    const float4 v = *reinterpret_cast<const float4*>(p);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
}
__device__ __forceinline__ void load4(const bf16_t* p, float (&x)[4]) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    x[0] = bf16_to_f32(v.x & 0xffffu); x[1] = bf16_to_f32(v.x >> 16);
    x[2] = bf16_to_f32(v.y & 0xffffu); x[3] = bf16_to_f32(v.y >> 16);
}
__device__ __forceinline__ void store4(float* p, const float (&x)[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void store4(bf16_t* p, const float (&x)[4]) {
    uint2 v;
    v.x = f32_to_bf16(x[0]) | ((uint32_t)f32_to_bf16(x[1]) << 16);
    v.y = f32_to_bf16(x[2]) | ((uint32_t)f32_to_bf16(x[3]) << 16);
    *reinterpret_cast<uint2*>(p) = v;
}

// float64 -> bf16 in one rounding (nearest, ties to even).  Normal range:
// round the double's 52-bit fraction to bf16's 7 bits on the integer
// pattern; the result has 8 significant bits, so the conversion to fp32 is
// exact (or overflows to inf, as the rounding demands) and its upper half
// is the bf16 pattern.  Below 2^-126 bf16 is subnormal with the fixed
// quantum 2^-133: x * 2^133 is rounded to an integer instead.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
    if (x != x) return 0x7fc0;
    if (fabs(x) < 0x1p-126) {
        const double r = rint(x * 0x1p133) * 0x1p-133;
        return static_cast<uint16_t>(__float_as_uint(static_cast<float>(r)) >> 16);
    }
    uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
    u += 0x0FFFFFFFFFFFull + ((u >> 45) & 1ull);
    u &= ~0x1FFFFFFFFFFFull;
    return static_cast<uint16_t>(__float_as_uint(static_cast<float>(__longlong_as_double((long long)u))) >> 16);
}
// Rotate 4 pairs (x0[e], x1[e]) by the angles of cos/sin cs[e], sn[e]:
// x0 cos - x1 sin goes to p[e], x1 cos + x0 sin to p[half + e], each
// computed in float64 and rounded once to the storage type.  One element at
// a time, so that few float64 values are live (the bf16 form packs its
// results as it goes): the kernel stays within 64 VGPRs.
__device__ __forceinline__ void rotate_store(float* p, int half, const float (&x0)[4], const float (&x1)[4],
                                             const double* cs, const double* sn) {
    float lo[4], hi[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        lo[e] = (float)((double)x0[e] * cs[e] - (double)x1[e] * sn[e]);
        hi[e] = (float)((double)x1[e] * cs[e] + (double)x0[e] * sn[e]);
    }
    *reinterpret_cast<float4*>(p) = make_float4(lo[0], lo[1], lo[2], lo[3]);
    *reinterpret_cast<float4*>(p + half) = make_float4(hi[0], hi[1], hi[2], hi[3]);
}
__device__ __forceinline__ void rotate_store(bf16_t* p, int half, const float (&x0)[4], const float (&x1)[4],
                                             const double* cs, const double* sn) {
    uint32_t lo[2] = {0u, 0u}, hi[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t sh = 16u * (e & 1);
        lo[e >> 1] |= (uint32_t)f64_to_bf16((double)x0[e] * cs[e] - (double)x1[e] * sn[e]) << sh;
        hi[e >> 1] |= (uint32_t)f64_to_bf16((double)x1[e] * cs[e] + (double)x0[e] * sn[e]) << sh;
    }
    *reinterpret_cast<uint2*>(p) = make_uint2(lo[0], lo[1]);
    *reinterpret_cast<uint2*>(p + half) = make_uint2(hi[0], hi[1]);
}

constexpr int kReorderThreads = 512;

template <typename T>
__global__ __launch_bounds__(kReorderThreads) void reorder_rope_append(ReorderArgs a) {
    const int i = blockIdx.x;   // logical slot
    const int b = blockIdx.y;
    const int W = a.W, D = a.D, half = D / 2;
    const int tid = threadIdx.x;
    const int lane = tid & 63;

    // Work items are 4 consecutive pairs (c .. c+3 with c+D/2 .. c+D/2+3) of
    // one head: Hq query heads, then Hkv key heads; value rows are copied in
    // 4-element pieces.
    const int qn = a.Hq * (half / 4), kn = a.Hkv * (half / 4), vn = a.Hkv * (D / 4);
    const int n_all = qn + kn + vn;
    const T* qs = static_cast<const T*>(a.q) + ((size_t)b * W + i) * a.Hq * D;
    const T* ks = static_cast<const T*>(a.k) + ((size_t)b * W + i) * a.Hkv * D;
    const T* vs = static_cast<const T*>(a.v) + ((size_t)b * W + i) * a.Hkv * D;

    // The rows of slot i depend on nothing else, so the first batch of
    // kMaxItems items per thread is loaded before the permutation, the page
    // and the angle table are known.  (Plain code, no lambdas: arrays
    // captured by a lambda were kept in scratch memory by the compiler.)
    constexpr int kMaxItems = 2;
    float x0[kMaxItems][4], x1[kMaxItems][4];
#pragma unroll
    for (int u = 0; u < kMaxItems; ++u) {
        const int it = tid + u * kReorderThreads;
        if (it >= n_all) continue;
        if (it < qn + kn) {
            const bool isq = it < qn;
            const int j = isq ? it : it - qn;
            const int hh = j / (half / 4), c = (j % (half / 4)) * 4;
            const T* src = (isq ? qs : ks) + (size_t)hh * D + c;
            load4(src, x0[u]);
            load4(src + half, x1[u]);
        } else {
            const int j = it - qn - kn;
            load4(vs + (size_t)j * 4, x0[u]);
        }
    }

    // Every wave derives the physical row of slot i by itself from two
    // ballots and a prefix popcount: no LDS, no barrier.
    const bool in = lane < W;
    const int f = in ? a.filled[(size_t)b * W + lane] : 0;
    const int p_lane = in ? a.pos[(size_t)b * W + lane] : 0;
    const int L = a.ctx_len[b];
    const uint64_t fm = __ballot(in && f != 0);
    const uint64_t mm = __ballot(in && f == 0);
    const uint64_t below = i == 0 ? 0ull : ((1ull << i) - 1ull);
    const int n_obs = __popcll(fm);
    const int r = ((fm >> i) & 1ull) ? __popcll(fm & below) : n_obs + __popcll(mm & below);
    const int p = __shfl(p_lane, i);

    // cos/sin of the D/2 pair angles, float64, once per work-group
    __shared__ double s_cs[64], s_sn[64];
    if (tid < half) {
        double sn, cs;
        sincos((double)p * exp2(-(2.0 * tid / D) * a.log2_base), &sn, &cs);
        s_cs[tid] = cs;
        s_sn[tid] = sn;
    }

    // The window's tokens L .. L+W-1 span at most W/16 + 2 pages: their
    // block-table entries are read as soon as L is known, one per lane.
    const bool ctx_ok = L >= 0 && (int64_t)L + W <= (int64_t)a.max_pages * kPage;
    int page = -1;
    {
        const int fp = ctx_ok ? L / kPage : 0;
        const int npg = ctx_ok ? (L + W - 1) / kPage - fp + 1 : 0;
        const int pg_lane = lane < npg ? a.block_table[(size_t)b * a.max_pages + fp + lane] : -1;
        if (ctx_ok) {
            page = __shfl(pg_lane, (L + r) / kPage - fp);
            if (page < 0 || page >= a.num_pages) page = -1;
        }
    }
    if (tid == 0) {
        a.perm[(size_t)b * W + r] = i;
        if (!ctx_ok) set_status(a.status, WEDLM_DEV_BAD_CTX);
        else if (page < 0) set_status(a.status, WEDLM_DEV_BAD_PAGE);
    }
    if (tid < 64 && i == 0) {
        const int p_prev = __shfl_up(p_lane, 1);
        const bool bad_pos = in && (p_lane < 0 || (lane > 0 && p_lane <= p_prev));
        if (__ballot(bad_pos) && lane == 0) set_status(a.status, WEDLM_DEV_BAD_POS);
    }
    const int t_row = L + r;
    const size_t row0 = page >= 0 ? ((size_t)page * a.Hkv) * kPage + (t_row % kPage) : 0;
    T* qd = static_cast<T*>(a.q_phys) + ((size_t)b * W + r) * a.Hq * D;
    T* kc = static_cast<T*>(a.k_cache);
    T* vc = static_cast<T*>(a.v_cache);
    __syncthreads();

    // Every later batch loads all its items before using any.
    for (int base = tid; base < n_all; base += kMaxItems * kReorderThreads) {
        if (base != tid)   // the first batch is already loaded
#pragma unroll
        for (int u = 0; u < kMaxItems; ++u) {
            const int it = base + u * kReorderThreads;
            if (it >= n_all) continue;
            if (it < qn + kn) {
                const bool isq = it < qn;
                const int j = isq ? it : it - qn;
                const int hh = j / (half / 4), c = (j % (half / 4)) * 4;
                const T* src = (isq ? qs : ks) + (size_t)hh * D + c;
                load4(src, x0[u]);
                load4(src + half, x1[u]);
            } else {
                const int j = it - qn - kn;
                load4(vs + (size_t)j * 4, x0[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < kMaxItems; ++u) {
            const int it = base + u * kReorderThreads;
            if (it >= n_all || (it >= qn && page < 0)) continue;   // no cache row without a page
            if (it < qn + kn) {
                const bool isq = it < qn;
                const int j = isq ? it : it - qn;
                const int hh = j / (half / 4), c = (j % (half / 4)) * 4;
                T* dst = isq ? qd + (size_t)hh * D + c : kc + (row0 + (size_t)hh * kPage) * D + c;
                rotate_store(dst, half, x0[u], x1[u], s_cs + c, s_sn + c);
            } else {
                const int j = it - qn - kn;
                const int g = j / (D / 4), d = (j % (D / 4)) * 4;
                store4(vc + (row0 + (size_t)g * kPage) * D + d, x0[u]);
            }
        }
    }
}

hipError_t launch_reorder(const ReorderArgs& a, int dtype, hipStream_t stream) {
    dim3 grid(a.W, a.B), block(kReorderThreads);
    if (dtype == WEDLM_F32)
        hipLaunchKernelGGL(reorder_rope_append<float>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(reorder_rope_append<bf16_t>, grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace wedlm
