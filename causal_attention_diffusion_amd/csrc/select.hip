// select.hip -- per-slot confidence over the vocabulary, commit of the
// leading filled run, the distance-penalised fill rule (Eq. 11) and window
// refill for one WeDLM decode step.
//
// Pages: "WeDLM: Reconciling Diffusion Language Models with Standard Causal
// Attention for Fast Inference", paper-summary page, "Method" (inference
// paragraph: commit the leftmost contiguous filled run, fill masks ranked by
// H~_j = H_j + alpha * d_j with d_j the distance to the leftmost remaining
// mask, refill the freed slots with masks) and "Key claims" (paper sec.
// 5.2); ICML abstract (a growing left-to-right committed prefix, fixed
// window).
//
// One launch.  Work-group (b, j, part) streams part `part` of the logits
// row of slot j when that slot is masked (rows of filled slots are never
// read): per thread an online (max, first argmax, S = sum e^{z-m},
// T = sum (z-m) e^{z-m}) over 16-byte loads, then a wave/LDS merge, and the
// partial is stored in the workspace.  Every work-group of sequence b then
// bumps b's arrival counter; the last one to arrive merges the row partials
// (H = ln S - T/S) and one wave, one lane per slot, runs commit / select /
// refill with ballots and shuffles, and puts the counter back to zero.
#include "kernels.hpp"

namespace wedlm {


struct Stat {
    float m;
    int a;
    float s, t;
};

// Merge two partial statistics (either may be empty: s == 0).
__device__ __forceinline__ Stat merge(const Stat& x, const Stat& y) {
    if (y.s == 0.f) return x;
    if (x.s == 0.f) return y;
    Stat o;
    o.m = fmaxf(x.m, y.m);
    o.a = x.m > y.m ? x.a : (y.m > x.m ? y.a : min(x.a, y.a));
    const float dx = x.m - o.m, dy = y.m - o.m;
    const float ex = exp2f(dx * kLog2e), ey = exp2f(dy * kLog2e);
    o.s = x.s * ex + y.s * ey;
    o.t = ex * (x.t + dx * x.s) + ey * (y.t + dy * y.s);
    return o;
}

__device__ __forceinline__ void accum(Stat& st, float z, int idx) {
    if (z > st.m) {
        if (st.s != 0.f) {
            const float dm = st.m - z;
            const float sc = exp2f(dm * kLog2e);
            st.t = sc * (st.t + dm * st.s);
            st.s *= sc;
        }
        st.m = z;
        st.a = idx;
    }
    const float u = z - st.m;
    const float e = exp2f(u * kLog2e);
    st.s += e;
    st.t += u * e;
}

__device__ __forceinline__ Stat shfl_xor_stat(const Stat& x, int mask) {
    Stat o;
    o.m = __shfl_xor(x.m, mask);
    o.a = __shfl_xor(x.a, mask);
    o.s = __shfl_xor(x.s, mask);
    o.t = __shfl_xor(x.t, mask);
    return o;
}

template <bool VEC>
__global__ __launch_bounds__(256) void vocab_select_commit(SelectArgs a) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int row = blockIdx.x / a.nparts;  // b * W + j
    const int part = blockIdx.x - row * a.nparts;
    const int b = row / a.W;

    __shared__ Stat s_red[4];
    __shared__ int s_last;

    const bool masked = a.filled[row] == 0;
    if (masked) {
        const int beg = part * a.part_len;
        const int end = min(a.V, beg + a.part_len);
        const float* z = a.logits + (size_t)row * a.V;
        Stat st{-INFINITY, 0x7fffffff, 0.f, 0.f};
        if constexpr (VEC) {
            // beg is a multiple of 4 (part_len is), V % 4 == 0
            const float4* z4 = reinterpret_cast<const float4*>(z);
            const int n4 = (end - beg) / 4;
            const int b4 = beg / 4;
            int i = tid;
            for (; i + 3 * 256 < n4; i += 4 * 256) {
                float4 v0 = z4[b4 + i], v1 = z4[b4 + i + 256], v2 = z4[b4 + i + 512], v3 = z4[b4 + i + 768];
                const int base = (b4 + i) * 4;
                accum(st, v0.x, base); accum(st, v0.y, base + 1); accum(st, v0.z, base + 2); accum(st, v0.w, base + 3);
                accum(st, v1.x, base + 1024); accum(st, v1.y, base + 1025); accum(st, v1.z, base + 1026); accum(st, v1.w, base + 1027);
                accum(st, v2.x, base + 2048); accum(st, v2.y, base + 2049); accum(st, v2.z, base + 2050); accum(st, v2.w, base + 2051);
                accum(st, v3.x, base + 3072); accum(st, v3.y, base + 3073); accum(st, v3.z, base + 3074); accum(st, v3.w, base + 3075);
            }
            for (; i < n4; i += 256) {
                float4 v0 = z4[b4 + i];
                const int base = (b4 + i) * 4;
                accum(st, v0.x, base); accum(st, v0.y, base + 1); accum(st, v0.z, base + 2); accum(st, v0.w, base + 3);
            }
        } else {
            for (int i = beg + tid; i < end; i += 256) accum(st, z[i], i);
        }
        // Each thread visits its indices in increasing order, so the strict
        // '>' in accum keeps the first index of a tied maximum; merge() takes
        // the lower index across threads.
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) st = merge(st, shfl_xor_stat(st, off));
        if (lane == 0) s_red[wv] = st;
        __syncthreads();
        if (tid == 0) {
            Stat o = s_red[0];
            for (int k = 1; k < 4; ++k) o = merge(o, s_red[k]);
            a.part[(size_t)row * a.nparts + part] = make_float4(o.m, __int_as_float(o.a), o.s, o.t);
        }
    }

    if (tid == 0) {
        __threadfence();
        const uint32_t total = (uint32_t)a.W * a.nparts;
        const uint32_t old = __hip_atomic_fetch_add(&a.counters[b], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (old == total - 1);
    }
    __syncthreads();
    if (!s_last || wv != 0) return;
    __threadfence();

    // ---- last arrival for sequence b: commit / select / refill (one wave)
    const int W = a.W;
    const int j = lane;
    const bool in = j < W;
    const size_t sj = (size_t)b * W + j;
    int tk = in ? a.tok[sj] : a.mask_id;
    int f = in ? a.filled[sj] : 1;
    const uint64_t fmask = __ballot(in && f != 0);
    const int k = ~fmask ? (int)__builtin_ctzll(~fmask) : 64;  // leading run of filled slots (<= W)
    const bool msk = in && f == 0;
    float H = -1.f;
    int am = -1;
    if (msk) {
        Stat o{-INFINITY, 0x7fffffff, 0.f, 0.f};
        for (int p = 0; p < a.nparts; ++p) {
            const float4 v = a.part[sj * a.nparts + p];
            Stat x{v.x, __float_as_int(v.y), v.z, v.w};
            o = merge(o, x);
        }
        am = o.a;
        H = logf(o.s) - o.t / o.s;
    }
    const uint64_t mmask = __ballot(msk);
    bool sel = false;
    if (mmask) {
        const int j0 = (int)__builtin_ctzll(mmask);
        const float Ht = msk ? fmaf(a.alpha, (float)(j - j0), H) : INFINITY;
        sel = msk && Ht < a.tau;
        if (__ballot(sel) == 0) {
            // argmin of Ht over masked slots, lowest slot on ties
            float bv = Ht;
            int bj = msk ? j : 0x7fffffff;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) {
                const float ov = __shfl_xor(bv, off);
                const int oj = __shfl_xor(bj, off);
                if (ov < bv || (ov == bv && oj < bj)) { bv = ov; bj = oj; }
            }
            sel = (j == bj);
        }
    }
    if (in) {
        a.committed[sj] = j < k ? tk : -1;
        if (a.argmax_out) a.argmax_out[sj] = am;
        if (a.entropy_out) a.entropy_out[sj] = H;
    }
    if (sel) { tk = am; f = 1; }
    // refill: shift left by k, masks enter on the right
    const int src = j + k;
    const int tk_s = __shfl(tk, src < 64 ? src : 0);
    const int f_s = __shfl(f, src < 64 ? src : 0);
    const int L = a.ctx_len[b];
    if (in) {
        const bool keep = src < W;
        a.tok[sj] = keep ? tk_s : a.mask_id;
        a.filled[sj] = keep ? (uint8_t)f_s : (uint8_t)0;
        a.pos[sj] = L + k + j;
    }
    if (lane == 0) {
        a.n_commit[b] = k;
        a.ctx_len[b] = L + k;
        a.counters[b] = 0u;
    }
}

hipError_t launch_select(const SelectArgs& a, hipStream_t st) {
    dim3 grid((unsigned)(a.B * a.W * a.nparts)), block(256);
    const bool vec = (a.V % 4 == 0) && (a.part_len % 4 == 0) &&
                     (reinterpret_cast<uintptr_t>(a.logits) % 16 == 0);
    if (vec)
        hipLaunchKernelGGL(vocab_select_commit<true>, grid, block, 0, st, a);
    else
        hipLaunchKernelGGL(vocab_select_commit<false>, grid, block, 0, st, a);
    return hipGetLastError();
}

}  // namespace wedlm
