// select.hpp -- the bodies of the select step's two kernels as device
// functions of (unit, thread), so that the plain launches (select.hip) and
// the fused decode-step launches (reorder.hip, attn.hip) run the same code.
//
// Pages: "WeDLM: Reconciling Diffusion Language Models with Standard Causal
// Attention for Fast Inference", paper-summary page, "Method" (inference
// paragraph: commit the leftmost contiguous filled run, fill masks ranked by
// H~_j = H_j + alpha * d_j with d_j the distance to the leftmost remaining
// mask, refill the freed slots with masks) and "Key claims" (paper sec.
// 5.2); ICML abstract (a growing left-to-right committed prefix, fixed
// window).
#pragma once

#include "kernels.hpp"
#include "stats.hpp"

namespace wedlm {

constexpr int kVecPerThread = 16;  // float4 loads per thread per full part (all in flight together)
constexpr int kVocabThreads = 256; // threads of one vocabulary unit

// Vocabulary statistics of one (row, part) unit by 256 threads t = 0..255:
// part `part` of the logits row of slot `row` when that slot is masked (rows
// of filled slots are never read).  Per thread an online (max, first
// argmax, S = sum 2^u, T = sum u 2^u with u = (z - max) log2 e) over 16-byte
// loads issued 16 at a time, then a wave merge into s_red[4] and, after the
// one barrier every thread of the work-group reaches (so several units may
// share a work-group), thread 0's merge writes the row-part partial.
// `valid` false: the unit is padding and only takes part in the barrier.
template <bool VEC>
__device__ __forceinline__ void vocab_unit(const SelectArgs& a, int unit, bool valid, int t, Stat* s_red) {
    const int lane = t & 63;
    const int wv = t >> 6;
    const int row = valid ? unit / a.nparts : 0;  // b * W + j
    const int part = unit - row * a.nparts;
    const bool masked = valid && a.filled[row] == 0;
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
                const int i = t + k * kVocabThreads;
                v[k] = i < n4 ? __builtin_nontemporal_load(z4 + b4 + i) : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            }
            accum_vec(st, v, (b4 + t) * 4);
        } else {
            for (int i = beg + t; i < end; i += kVocabThreads) accum_one(st, z[i], i);
        }
        // Each thread visits its indices in increasing order, so the strict
        // '>' in accum keeps the first index of a tied maximum; merge() takes
        // the lower index across threads.
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) st = merge(st, shfl_xor_stat(st, off));
        if (lane == 0) s_red[wv] = st;
    }
    __syncthreads();
    if (masked && t == 0) {
        Stat o = s_red[0];
        for (int k = 1; k < 4; ++k) o = merge(o, s_red[k]);
        a.part[(size_t)row * a.nparts + part] = make_float4(o.m, __int_as_float(o.a), o.s, o.t);
    }
}

// Commit / Eq. 11 select / refill of sequence b by one wave (one lane per
// slot), after every row partial of the sequence is in a.part.  Wave-level
// only (ballots and shuffles, no LDS, no barrier), so any wave of a launch
// can run it.
__device__ __forceinline__ void commit_seq(const SelectArgs& a, int b, int lane) {
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

// The vocabulary pass reads 16-byte vectors when the row length, the part
// length and the logits base allow it.
inline bool vocab_vec(const SelectArgs& a) {
    return (a.V % 4 == 0) && (a.part_len % 4 == 0) && (reinterpret_cast<uintptr_t>(a.logits) % 16 == 0);
}

}  // namespace wedlm
