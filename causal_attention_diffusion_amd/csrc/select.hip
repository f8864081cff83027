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
// Two launches.  vocab_stats: work-group (b, j, part) streams part `part` of
// the logits row of slot j when that slot is masked (rows of filled slots
// are never read): per thread an online (max, first argmax, S = sum 2^u,
// T = sum u 2^u with u = (z - max) log2 e) over 16-byte loads issued 16 at a
// time, then a wave/LDS merge, and the row-part partial goes to the
// workspace.  commit_select_refill: one wave per sequence, one lane per
// slot, merges its rows' partials (H = ln S - ln2 T/S) and runs commit /
// select / refill with ballots and shuffles.  The kernel boundary orders
// the two; an in-kernel last-arrival scheme would need an agent-scope
// release fence per work-group, which writes back L2 and cost more than a
// second launch.
#include "kernels.hpp"
#include "stats.hpp"

namespace wedlm {

constexpr int kVecPerThread = 16;  // float4 loads per thread per full part (all in flight together)


template <bool VEC>
__global__ __launch_bounds__(256) void vocab_stats(SelectArgs a) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int row = blockIdx.x / a.nparts;  // b * W + j
    const int part = blockIdx.x - row * a.nparts;

    __shared__ Stat s_red[4];

    const bool masked = a.filled[row] == 0;
    if (masked) {
        const int beg = part * a.part_len;
        const int end = min(a.V, beg + a.part_len);
        const float* z = a.logits + (size_t)row * a.V;
        Stat st{-INFINITY, 0x7fffffff, 0.f, 0.f};
        if constexpr (VEC) {
            // part_len and beg are multiples of 4 and V % 4 == 0; a part is at
            // most kVecPerThread 16-byte loads per thread, all issued up front
            // (non-temporal: every logit is read once), -inf past its end
            const f32x4* z4 = reinterpret_cast<const f32x4*>(z);
            const int n4 = (end - beg) / 4;
            const int b4 = beg / 4;
            f32x4 v[kVecPerThread];
#pragma unroll
            for (int k = 0; k < kVecPerThread; ++k) {
                const int i = tid + k * 256;
                v[k] = i < n4 ? __builtin_nontemporal_load(z4 + b4 + i) : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            }
            accum_vec(st, v, (b4 + tid) * 4);
        } else {
            for (int i = beg + tid; i < end; i += 256) accum_one(st, z[i], i);
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
}

// Commit / Eq. 11 select / refill of one sequence per 64-thread work-group
// (one lane per slot), after vocab_stats has written every row partial.
__global__ __launch_bounds__(64) void commit_select_refill(SelectArgs a) {
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const int W = a.W;
    const int j = lane;
    const bool in = j < W;
    const size_t sj = (size_t)b * W + j;
    const int L = a.ctx_len[b];
    int tk = in ? a.tok[sj] : a.mask_id;
    int f = in ? a.filled[sj] : 1;
    // The row partials are read for every slot in the window, 16 at a time
    // with all loads in flight, so that they do not wait for the flags; only
    // the masked slots' (written by vocab_stats) are used.
    Stat o{-INFINITY, 0x7fffffff, 0.f, 0.f};
    if (in) {
        const float4* pp = a.part + sj * a.nparts;
        for (int p0 = 0; p0 < a.nparts; p0 += 16) {
            float4 v[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) v[q] = p0 + q < a.nparts ? pp[p0 + q] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const Stat x{v[q].x, __float_as_int(v[q].y), v[q].z, v[q].w};  // s == 0: empty, skipped
                o = merge(o, x);
            }
        }
    }
    const uint64_t fmask = __ballot(in && f != 0);
    const int k = ~fmask ? (int)__builtin_ctzll(~fmask) : 64;  // leading run of filled slots (<= W)
    const bool msk = in && f == 0;
    float H = -1.f;
    int am = -1;
    if (msk) {
        am = o.a;
        H = logf(o.s) - 0.69314718055994531f * (o.t / o.s);
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
    if (in) {
        const bool keep = src < W;
        a.tok[sj] = keep ? tk_s : a.mask_id;
        a.filled[sj] = keep ? (uint8_t)f_s : (uint8_t)0;
        a.pos[sj] = L + k + j;
    }
    if (lane == 0) {
        a.n_commit[b] = k;
        a.ctx_len[b] = L + k;
        // prefix cacheability: N_new counts committed tokens, N_total the
        // window slots this step processed (one wave per sequence, so the
        // update needs no atomics)
        if (a.counters) {
            a.counters[2 * b] += k;
            a.counters[2 * b + 1] += W;
        }
    }
}

hipError_t launch_select(const SelectArgs& a, hipStream_t st) {
    dim3 grid((unsigned)(a.B * a.W * a.nparts)), block(256);
    const bool vec = (a.V % 4 == 0) && (a.part_len % 4 == 0) &&
                     (reinterpret_cast<uintptr_t>(a.logits) % 16 == 0);
    if (vec)
        hipLaunchKernelGGL(vocab_stats<true>, grid, block, 0, st, a);
    else
        hipLaunchKernelGGL(vocab_stats<false>, grid, block, 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_commit(a, st);
}

hipError_t launch_commit(const SelectArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(commit_select_refill, dim3((unsigned)a.B), dim3(64), 0, st, a);
    return hipGetLastError();
}

}  // namespace wedlm
