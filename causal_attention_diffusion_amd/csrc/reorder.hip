// reorder.hip -- Topological Reordering, RoPE at logical positions and KV
// append for one WeDLM decode step.
//
// Pages: "WeDLM: Reconciling Diffusion Language Models with Standard Causal
// Attention for Fast Inference", paper-summary page, "Key claims" (paper
// sec. 4.1, Eq. 5-6: observed tokens go to the physical front, RoPE keeps
// their logical positions) and "Method" (inference paragraph: the window is
// reordered with filled tokens first before the causal pass on the cache).
//
// One work-group per (run of SPW logical slots, sequence b): one slot for a
// decode window, four for the thousands of one-block windows of a
// Dual-Stream pass.  It loads the rows of its slots at once, and meanwhile
// each wave derives the slots' physical rows with two ballots (filled /
// masked masks) and prefix popcounts: slot i lands at r = popc(filled below
// i) if filled, else n_obs + popc(masked below i).  The work-group then
// rotates the Hq query heads and Hkv key heads at each slot's logical
// position into physical row r and writes the key/value rows into the paged
// cache at token ctx_len[b] + r.
// The work is tiny (B*W*(Hq+2Hkv)*D elements) and latency-bound; angles and
// rotations are float64 so that positions up to 2^31 keep full accuracy.
// The same body also runs inside the fused decode step's front launch
// (beside the vocabulary pass) and, for the synthetic decoder, straight from
// the q/k/v projection's split partials.
#include "select.hpp"

namespace wedlm {


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

// Raw 4-element pieces as loaded (bf16 stays packed until it is used, so a
// thread can hold more pieces in flight in the same registers).
template <typename T> struct Piece;
template <> struct Piece<float> {
    using type = float4;
    __device__ static type load(const float* p) { return *reinterpret_cast<const float4*>(p); }
    __device__ static void unpack(const type& v, float (&x)[4]) { x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w; }
    __device__ static void store(float* p, const type& v) { *reinterpret_cast<float4*>(p) = v; }
};
template <> struct Piece<bf16_t> {
    using type = uint2;
    __device__ static type load(const bf16_t* p) { return *reinterpret_cast<const uint2*>(p); }
    __device__ static void unpack(const type& v, float (&x)[4]) {
        x[0] = bf16_to_f32(v.x & 0xffffu); x[1] = bf16_to_f32(v.x >> 16);
        x[2] = bf16_to_f32(v.y & 0xffffu); x[3] = bf16_to_f32(v.y >> 16);
    }
    __device__ static void store(bf16_t* p, const type& v) { *reinterpret_cast<uint2*>(p) = v; }
};

// SPW consecutive logical slots of one sequence per work-group: one for a
// decode window (a few dozen slots: every slot gets its own work-group and
// CU), four for the thousands of slots of a Dual-Stream pass (a quarter of
// the work-groups, each with four times the loads in flight).
// Projection form: four consecutive columns n .. n+3 of row m of the stacked
// q/k/v projection, summed over the split-K partials in split order and
// rounded to bf16, exactly as the projection's own finish would store them.
// The partials are loaded four splits at a time (all four in flight) and
// added in split order.
__device__ __forceinline__ uint2 part_bf16x4(const ReorderArgs& a, size_t m, int n) {
    const float* p = a.part + m * a.part_N + n;
    const size_t plane = (size_t)a.B * a.W * a.part_N;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = 0; s0 < a.part_S; s0 += 4) {
        float4 w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (s0 + j < a.part_S) w[j] = *reinterpret_cast<const float4*>(p + (size_t)(s0 + j) * plane);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (s0 + j < a.part_S) v = s0 + j == 0 ? w[0] : add4(v, w[j]);
    }
    return pack_bf16x4(v);
}

template <typename T, int SPW, int NT, bool FROM_PART = false>
__device__ __forceinline__ void reorder_slots(const ReorderArgs& a, int bx, int b) {
    static_assert(!FROM_PART || sizeof(T) == 2, "the projection form is bf16");
    static_assert(NT >= 4 * 64, "the angle table takes up to four slots x 64 threads");
    using P = Piece<T>;
    const int i0 = bx * SPW;           // first logical slot
    const int W = a.W, D = a.D, half = D / 2;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int ns = min(SPW, W - i0);   // slots of this work-group

    // Work items are 4 consecutive pairs (c .. c+3 with c+D/2 .. c+D/2+3) of
    // one head of one slot: Hq query heads, then Hkv key heads; value rows
    // are copied in 4-element pieces.
    const int qn = a.Hq * (half / 4), kn = a.Hkv * (half / 4), vn = a.Hkv * (D / 4);
    const int n_all = qn + kn + vn;
    const int n_tot = ns * n_all;
    const size_t row_first = (size_t)b * W + i0;

    // The slots' rows depend on nothing else, so the first batch of
    // kMaxItems items per thread is loaded before the permutation, the pages
    // and the angle tables are known.  (Plain code, no lambdas: arrays
    // captured by a lambda were kept in scratch memory by the compiler.)
    constexpr int kMaxItems = SPW == 1 ? 1024 / NT : 6;
    typename P::type r0[kMaxItems], r1[kMaxItems];
#pragma unroll
    for (int u = 0; u < kMaxItems; ++u) {
        const int it = tid + u * NT;
        if (it >= n_tot) continue;
        const int sl = it / n_all, jj = it - sl * n_all;
        const size_t row = row_first + sl;
        if (jj < qn + kn) {
            const bool isq = jj < qn;
            const int j = isq ? jj : jj - qn;
            const int hh = j / (half / 4), c = (j % (half / 4)) * 4;
            if constexpr (FROM_PART) {
                const int n = (isq ? 0 : a.Hq * D) + hh * D + c;
                r0[u] = part_bf16x4(a, row, n);
                r1[u] = part_bf16x4(a, row, n + half);
            } else {
                const T* src = isq ? static_cast<const T*>(a.q) + (row * a.Hq + hh) * D + c
                                   : static_cast<const T*>(a.k) + (row * a.Hkv + hh) * D + c;
                r0[u] = P::load(src);
                r1[u] = P::load(src + half);
            }
        } else {
            const int j = jj - qn - kn;
            if constexpr (FROM_PART)
                r0[u] = part_bf16x4(a, row, (a.Hq + a.Hkv) * D + j * 4);
            else
                r0[u] = P::load(static_cast<const T*>(a.v) + row * a.Hkv * D + (size_t)j * 4);
        }
    }

    // Every wave derives the physical rows of its slots by itself from two
    // ballots and prefix popcounts: slot i lands at r = popc(filled below i)
    // if filled, else n_obs + popc(masked below i).  No LDS, no barrier.
    const bool in = lane < W;
    const int f = in ? a.filled[(size_t)b * W + lane] : 0;
    const int p_lane = in ? a.pos[(size_t)b * W + lane] : 0;
    const int L = a.ctx_len[b];
    const uint64_t fm = __ballot(in && f != 0);
    const uint64_t mm = __ballot(in && f == 0);
    const int n_obs = __popcll(fm);
    int rr[SPW], pp[SPW];
#pragma unroll
    for (int sl = 0; sl < SPW; ++sl) {
        const int i = min(i0 + sl, W - 1);
        const uint64_t below = i == 0 ? 0ull : ((1ull << i) - 1ull);
        rr[sl] = ((fm >> i) & 1ull) ? __popcll(fm & below) : n_obs + __popcll(mm & below);
        pp[sl] = __shfl(p_lane, i);
    }

    // cos/sin of the D/2 pair angles of every slot, float64, once per
    // work-group
    __shared__ double s_cs[SPW][64], s_sn[SPW][64];
    if (tid < ns * half) {
        const int sl = tid / half, t = tid - sl * half;
        int p = pp[0];
#pragma unroll
        for (int k = 1; k < SPW; ++k) p = sl == k ? pp[k] : p;
        double sn, cs;
        sincos((double)p * exp2(-(2.0 * t / D) * a.log2_base), &sn, &cs);
        s_cs[sl][t] = cs;
        s_sn[sl][t] = sn;
    }

    // The window's tokens L .. L+W-1 span at most W/16 + 2 pages: their
    // block-table entries are read as soon as L is known, one per lane.
    const bool ctx_ok = L >= 0 && (int64_t)L + W <= (int64_t)a.max_pages * kPage;
    size_t row0[SPW];     // cache row (page, head 0, offset) of each slot's token, or none
    bool has_page[SPW];
    bool bad_page = false;
    {
        const int fp = ctx_ok ? L / kPage : 0;
        const int npg = ctx_ok ? (L + W - 1) / kPage - fp + 1 : 0;
        const int pg_lane = lane < npg ? a.block_table[(size_t)b * a.max_pages + fp + lane] : -1;
#pragma unroll
        for (int sl = 0; sl < SPW; ++sl) {
            int page = -1;
            if (ctx_ok) {
                page = __shfl(pg_lane, (L + rr[sl]) / kPage - fp);
                if (page < 0 || page >= a.num_pages) page = -1;
            }
            has_page[sl] = page >= 0;
            if (sl < ns && page < 0) bad_page = true;
            const int t_row = L + rr[sl];
            row0[sl] = page >= 0 ? ((size_t)page * a.Hkv) * kPage + (t_row % kPage) : 0;
        }
    }
    if (tid < ns) {
        int r = rr[0];
#pragma unroll
        for (int k = 1; k < SPW; ++k) r = tid == k ? rr[k] : r;
        a.perm[(size_t)b * W + r] = i0 + tid;
    }
    if (tid == 0) {
        if (!ctx_ok) set_status(a.status, WEDLM_DEV_BAD_CTX);
        else if (bad_page) set_status(a.status, WEDLM_DEV_BAD_PAGE);
    }
    if (tid < 64 && i0 == 0) {
        const int p_prev = __shfl_up(p_lane, 1);
        const bool bad_pos = in && (p_lane < 0 || (lane > 0 && p_lane <= p_prev));
        if (__ballot(bad_pos) && lane == 0) set_status(a.status, WEDLM_DEV_BAD_POS);
    }
    T* kc = static_cast<T*>(a.k_cache);
    T* vc = static_cast<T*>(a.v_cache);
    __syncthreads();

    // Every later batch loads all its items before using any.
    for (int base = tid; base < n_tot; base += kMaxItems * NT) {
        if (base != tid)   // the first batch is already loaded
#pragma unroll
        for (int u = 0; u < kMaxItems; ++u) {
            const int it = base + u * NT;
            if (it >= n_tot) continue;
            const int sl = it / n_all, jj = it - sl * n_all;
            const size_t row = row_first + sl;
            if (jj < qn + kn) {
                const bool isq = jj < qn;
                const int j = isq ? jj : jj - qn;
                const int hh = j / (half / 4), c = (j % (half / 4)) * 4;
                if constexpr (FROM_PART) {
                    const int n = (isq ? 0 : a.Hq * D) + hh * D + c;
                    r0[u] = part_bf16x4(a, row, n);
                    r1[u] = part_bf16x4(a, row, n + half);
                } else {
                    const T* src = isq ? static_cast<const T*>(a.q) + (row * a.Hq + hh) * D + c
                                       : static_cast<const T*>(a.k) + (row * a.Hkv + hh) * D + c;
                    r0[u] = P::load(src);
                    r1[u] = P::load(src + half);
                }
            } else {
                const int j = jj - qn - kn;
                if constexpr (FROM_PART)
                    r0[u] = part_bf16x4(a, row, (a.Hq + a.Hkv) * D + j * 4);
                else
                    r0[u] = P::load(static_cast<const T*>(a.v) + row * a.Hkv * D + (size_t)j * 4);
            }
        }
#pragma unroll
        for (int u = 0; u < kMaxItems; ++u) {
            const int it = base + u * NT;
            if (it >= n_tot) continue;
            const int sl = it / n_all, jj = it - sl * n_all;
            int r = rr[0];
            size_t rw = row0[0];
            bool hp = has_page[0];
#pragma unroll
            for (int k = 1; k < SPW; ++k) {
                r = sl == k ? rr[k] : r;
                rw = sl == k ? row0[k] : rw;
                hp = sl == k ? has_page[k] : hp;
            }
            if (jj >= qn && !hp) continue;   // no cache row without a page
            if (jj < qn + kn) {
                const bool isq = jj < qn;
                const int j = isq ? jj : jj - qn;
                const int hh = j / (half / 4), c = (j % (half / 4)) * 4;
                T* dst = isq ? static_cast<T*>(a.q_phys) + (((size_t)b * W + r) * a.Hq + hh) * D + c
                             : kc + (rw + (size_t)hh * kPage) * D + c;
                float x0[4], x1[4];
                P::unpack(r0[u], x0);
                P::unpack(r1[u], x1);
                rotate_store(dst, half, x0, x1, &s_cs[sl][c], &s_sn[sl][c]);
            } else {
                const int j = jj - qn - kn;
                const int g = j / (D / 4), d = (j % (D / 4)) * 4;
                P::store(vc + (rw + (size_t)g * kPage) * D + d, r0[u]);
            }
        }
    }
}

template <typename T, int SPW>
__global__ __launch_bounds__(kReorderThreads) void reorder_rope_append(ReorderArgs a) {
    reorder_slots<T, SPW, kReorderThreads>(a, blockIdx.x, blockIdx.y);
}

// The decoder step's reorder straight from its [Wq; Wk; Wv] projection's
// split-K partials: the same slots, rotations and stores, with no separate
// launch to sum the partials into bf16 q, k and v first.
__global__ __launch_bounds__(kReorderThreads) void reorder_from_partials(ReorderArgs a) {
    reorder_slots<bf16_t, 1, kReorderThreads, true>(a, blockIdx.x, blockIdx.y);
}

// Front half of a fused decode step: the reorder's work-groups (first, one
// per run of slots of a sequence, 256 threads each here) and the vocabulary
// pass's (row, part) units, one per work-group as in vocab_stats, in one
// launch.  They share nothing: the reorder reads the flags, positions,
// q/k/v, block table and ctx_len and writes perm, q_phys and the window's
// cache rows; the vocabulary pass reads the flags and logits and writes its
// partials.  256-thread work-groups keep the vocabulary units at the
// occupancy of their own launch (a 512-thread form, two units per
// work-group, held fewer waves per CU and ran the units slower).
template <typename T, int SPW, bool VEC>
__global__ __launch_bounds__(kVocabThreads) void step_front(ReorderArgs r, SelectArgs s, int nx) {
    const int blk = blockIdx.x;
    const int nr = nx * r.B;
    if (blk < nr) {
        reorder_slots<T, SPW, kVocabThreads>(r, blk % nx, blk / nx);
    } else {
        __shared__ Stat s_red[4];
        vocab_unit<VEC>(s, blk - nr, true, threadIdx.x, s_red);
    }
}

// A Dual-Stream pass (thousands of slots) runs four slots per bf16
// work-group; a decode window keeps one per slot.
constexpr int kManySlots = 2048;

static int reorder_spw(const ReorderArgs& a, int dtype) {
    return dtype == WEDLM_BF16 && (int64_t)a.B * a.W >= kManySlots ? 4 : 1;
}

hipError_t launch_reorder(const ReorderArgs& a, int dtype, hipStream_t stream) {
    dim3 block(kReorderThreads);
    if (reorder_spw(a, dtype) == 4) {
        dim3 grid((a.W + 3) / 4, a.B);
        hipLaunchKernelGGL((reorder_rope_append<bf16_t, 4>), grid, block, 0, stream, a);
    } else if (dtype == WEDLM_F32) {
        hipLaunchKernelGGL((reorder_rope_append<float, 1>), dim3(a.W, a.B), block, 0, stream, a);
    } else {
        hipLaunchKernelGGL((reorder_rope_append<bf16_t, 1>), dim3(a.W, a.B), block, 0, stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_reorder_from_partials(const ReorderArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(reorder_from_partials, dim3(a.W, a.B), dim3(kReorderThreads), 0, stream, a);
    return hipGetLastError();
}

template <typename T, int SPW, bool VEC>
static hipError_t launch_front_t(const ReorderArgs& r, const SelectArgs& s, hipStream_t st) {
    const int nx = (r.W + SPW - 1) / SPW;
    const long units = (long)s.B * s.W * s.nparts;
    const long blocks = (long)nx * r.B + units;
    hipLaunchKernelGGL((step_front<T, SPW, VEC>), dim3((unsigned)blocks), dim3(kVocabThreads), 0, st, r, s, nx);
    return hipGetLastError();
}

hipError_t launch_step_front(const ReorderArgs& r, const SelectArgs& s, int dtype, hipStream_t st) {
    const bool vec = vocab_vec(s);
    if (reorder_spw(r, dtype) == 4)
        return vec ? launch_front_t<bf16_t, 4, true>(r, s, st) : launch_front_t<bf16_t, 4, false>(r, s, st);
    if (dtype == WEDLM_F32)
        return vec ? launch_front_t<float, 1, true>(r, s, st) : launch_front_t<float, 1, false>(r, s, st);
    return vec ? launch_front_t<bf16_t, 1, true>(r, s, st) : launch_front_t<bf16_t, 1, false>(r, s, st);
}

}  // namespace wedlm
