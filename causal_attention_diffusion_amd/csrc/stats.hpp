// stats.hpp -- online per-row vocabulary statistics (max, first argmax and
// the two exponential sums that give the softmax entropy), shared by the
// select kernels that read stored logits and the LM-head kernel that makes
// them on the fly.
//
// Pages: WeDLM paper-summary page, "Method" (inference paragraph: slots are
// ranked by the entropy H_j of their predictive distribution; the fill
// token is the most likely one).
#pragma once

#include "common.hpp"

namespace wedlm {

// Online statistics of a logits row slice: max m, first argmax a,
// S = sum 2^{u} and T = sum u 2^{u} with u = (z - m) * log2(e), so that the
// entropy in nats is H = ln S - ln(2) T / S.
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
    const float dx = (x.m - o.m) * kLog2e, dy = (y.m - o.m) * kLog2e;
    const float ex = __builtin_amdgcn_exp2f(dx), ey = __builtin_amdgcn_exp2f(dy);
    o.s = x.s * ex + y.s * ey;
    o.t = ex * fmaf(dx, x.s, x.t) + ey * fmaf(dy, y.s, y.t);
    return o;
}

// Move the reference maximum of st up to bm (new first argmax ba).
__device__ __forceinline__ void raise_max(Stat& st, float bm, int ba) {
    if (st.s != 0.f) {
        const float d = (st.m - bm) * kLog2e;
        const float sc = __builtin_amdgcn_exp2f(d);
        st.t = sc * fmaf(d, st.s, st.t);
        st.s *= sc;
    }
    st.m = bm;
    st.a = ba;
}

// Add exp terms of one value (its maximum is already folded into st.m).
__device__ __forceinline__ void add_term(float& s, float& t, float z, float m) {
    // (z - m) first: exact 0 at the maximum, so a row with one dominant
    // logit gets exactly S = 1, T = 0 there (H = 0 for a certain row).  The
    // clamp at -200 (2^-200 is 0 in fp32) keeps u * 2^u = 0 for -inf
    // logits and padding instead of -inf * 0.
    const float u = fmaxf((z - m) * kLog2e, -200.f);
    const float e = __builtin_amdgcn_exp2f(u);
    s += e;
    t = fmaf(u, e, t);
}

// Fold K 4-vectors (element j of v[k] has index base + 1024 k + j,
// increasing in visiting order) into st: one max test per batch.  Padding
// entries hold -inf: they never become the maximum and add 0 to S and T.
template <int K>
__device__ __forceinline__ void accum_vec(Stat& st, const f32x4 (&v)[K], int base) {
    float bm = fmaxf(fmaxf(v[0][0], v[0][1]), fmaxf(v[0][2], v[0][3]));
#pragma unroll
    for (int k = 1; k < K; ++k) bm = fmaxf(bm, fmaxf(fmaxf(v[k][0], v[k][1]), fmaxf(v[k][2], v[k][3])));
    if (bm > st.m) {
        int ba = 0x7fffffff;
#pragma unroll
        for (int k = K - 1; k >= 0; --k) {   // backwards, so the first match wins
            const int i0 = base + 1024 * k;
#pragma unroll
            for (int j = 3; j >= 0; --j)
                if (v[k][j] == bm) ba = i0 + j;
        }
        raise_max(st, bm, ba);
    }
    float s = 0.f, t = 0.f;
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
        for (int j = 0; j < 4; ++j) add_term(s, t, v[k][j], st.m);
    st.s += s;
    st.t += t;
}

__device__ __forceinline__ void accum_one(Stat& st, float z, int idx) {
    if (z > st.m) raise_max(st, z, idx);
    float s = 0.f, t = 0.f;
    add_term(s, t, z, st.m);
    st.s += s;
    st.t += t;
}

__device__ __forceinline__ Stat shfl_xor_stat(const Stat& x, int mask) {
    Stat o;
    o.m = __shfl_xor(x.m, mask);
    o.a = __shfl_xor(x.a, mask);
    o.s = __shfl_xor(x.s, mask);
    o.t = __shfl_xor(x.t, mask);
    return o;
}

}  // namespace wedlm
