// attn.hip -- fp32 windowed causal grouped-query attention of one WeDLM
// decode step over a paged prefix KV cache (gfx950, MFMA), the split-KV
// combine shared by the fp32 and bf16 kernels, and the fused decode step's
// back launch (the combine beside the commit / select / refill).
//
// Pages: "WeDLM: Reconciling Diffusion Language Models with Standard Causal
// Attention for Fast Inference", paper-summary page, "Key claims" (paper
// sec. 3.2: every masked slot must see all observed tokens; sec. 4.1: after
// the reordering a plain causal mask does this; sec. 5.2: a decode step is a
// causal pass of the window over the cached prefix) and risewithvishwas
// WeDLM page, "Attention Mechanism" (lower-triangular mask).
//
// Work decomposition.  For one (sequence b, KV head g) the M = W * (Hq/Hkv)
// query rows (physical window row r, group head) share every K/V byte, so
// they are packed into row tiles of RT = 32 * NW rows; wave w of a
// work-group owns rows [32w, 32w + 32) of its tile.  The key range
// [0, ctx_len + W) is cut into splits of split_keys keys, one work-group per
// (b, g, row tile, split); partial (O, m, l) of several splits are merged by
// attn_combine with the usual log-sum-exp rule.
//
// Per work-group the keys stream through LDS in chunks of 32 keys with a
// register-staged double buffer: 16-byte coalesced global loads of whole
// (page, head) blocks, paged through a block-table slice held in LDS.
//
// Tiles are transposed so that one lane owns one query row:
//   S^T[key][row] = K[key][:] . Q[row][:]       (v_mfma_f32_32x32x2f32:
//                                                 A = K from LDS, B = Q in VGPRs)
//   O^T[d][row]  += V^T[d][key] P^T[key][row]   (A = V from LDS, B = P from
//                                                 S^T's VGPRs)
// A lane's 16 outputs are 16 keys (or 16 d) of one row (lane % 32), so the
// online-softmax max/sum are in-lane plus one exchange with lane ^ 32, and
// the O rescale is in-lane.
//
// The bf16 kernels (attn_bf16.hip) use the same transposed tiling with
// direct global-to-LDS loads.
#include "select.hpp"

namespace wedlm {

template <int D, int NW>
struct AttnCfg {
    static constexpr int CHUNK = 32;           // keys per LDS chunk
    static constexpr int NT = 64 * NW;
    static constexpr int RT = 32 * NW;
    static constexpr int KS = D + 4;           // padded K row (floats): rows 16 B apart in bank space
    static constexpr int VS = D + 4;
    static constexpr int ROWP = D * 4 / 16;    // 16-byte pieces per key row
    static constexpr int PIECES = CHUNK * ROWP;
    static constexpr int PPT = PIECES / NT;    // pieces per thread per K (or V) chunk
    static constexpr int NDT = D / 32;
    static_assert(PIECES % NT == 0, "chunk must split evenly over the threads");
};

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void attn_split_f32(AttnArgs a) {
    using C = AttnCfg<D, NW>;
    constexpr int CHUNK = C::CHUNK;
    __shared__ __attribute__((aligned(16))) float s_k[2][CHUNK * C::KS];
    __shared__ __attribute__((aligned(16))) float s_v[2][CHUNK * C::VS];
    __shared__ int s_pages[kMaxSplitPages];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int hl = lane >> 5;   // lane half
    const int col = lane & 31;  // row within the wave's 32 (S^T / O^T column)

    // split-major order: every (sequence, KV head, row tile) gets its first
    // split dispatched before any second split, so the dispatcher hands the
    // remaining (equal-size) splits of long sequences to whichever CU frees
    // up first
    const int npid = a.B * a.Hkv * a.row_tiles;
    const int split = blockIdx.x / npid;
    const int pid = blockIdx.x - split * npid;
    const int rt = pid % a.row_tiles;
    const int bk = pid / a.row_tiles;
    const int kvh = bk % a.Hkv;
    const int b = bk / a.Hkv;

    int L = a.ctx_len[b];
    const bool ctx_ok = L >= 0 && L <= a.max_ctx && (int64_t)L + a.W <= (int64_t)a.max_pages * kPage;
    if (!ctx_ok) {
        if (tid == 0 && split == 0 && rt == 0 && kvh == 0) set_status(a.status, WEDLM_DEV_BAD_CTX);
        L = 0;
    }
    const int T_len = ctx_ok ? L + a.W : 0;
    const int sk = split_len(T_len, a.nsplit, a.split_keys, a.split_align);
    const int k_begin = split * sk;
    const int k_end = min(T_len, k_begin + sk);
    if (k_begin >= k_end && a.nsplit > 1) {
        // no key here: the split's rows get an empty partial (m = -inf, l = 0),
        // which attn_combine weighs zero without reading its O
        const size_t prow0 = ((size_t)pid * a.nsplit + split) * C::RT;
        for (int i = tid; i < C::RT; i += C::NT)
            if (rt * C::RT + i < a.M) a.part_ml[prow0 + i] = make_float2(-INFINITY, 0.f);
        return;
    }

    // block-table slice of this split
    const int p0 = k_begin / kPage;
    const int np = k_end > k_begin ? (k_end + kPage - 1) / kPage - p0 : 0;
    for (int i = tid; i < np; i += C::NT) {
        int pg = a.block_table[(size_t)b * a.max_pages + p0 + i];
        if (pg < 0 || pg >= a.num_pages) {
            set_status(a.status, WEDLM_DEV_BAD_PAGE);
            pg = -1;
        }
        s_pages[i] = pg;
    }

    // this lane's query row
    const int m = rt * C::RT + w * 32 + col;
    const bool row_ok = m < a.M;
    const int r = row_ok ? m / a.G : a.W;  // padding rows see every key (their q is 0)
    const int h = kvh * a.G + (row_ok ? m % a.G : 0);
    const int lim = L + r;                  // last visible key
    const size_t q_off = (((size_t)b * a.W + (row_ok ? r : 0)) * a.Hq + h) * D;

    // Q fragments (B operand of S^T = K Q^T), kept in VGPRs
    constexpr int NQ = D / 2;
    float qf[NQ];
    {
        const float* qp = static_cast<const float*>(a.q) + q_off + hl * (D / 2);
#pragma unroll
        for (int s = 0; s < NQ; ++s) qf[s] = row_ok ? qp[s] : 0.f;
    }

    f32x16 oacc[C::NDT];
#pragma unroll
    for (int i = 0; i < C::NDT; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[i][e] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    __syncthreads();  // s_pages ready

    const char* kbase = static_cast<const char*>(a.k_cache);
    const char* vbase = static_cast<const char*>(a.v_cache);
    uint4 kr[C::PPT], vr[C::PPT];

    auto load_chunk = [&](int c) {
        const int kb = k_begin + c * CHUNK;
#pragma unroll
        for (int i = 0; i < C::PPT; ++i) {
            const int piece = tid + i * C::NT;
            const int kc = piece / C::ROWP;
            const int pc = piece - kc * C::ROWP;
            const int t = kb + kc;
            int pg = -1;
            if (t < k_end) pg = s_pages[t / kPage - p0];
            if (pg >= 0) {
                const size_t off = ((((size_t)pg * a.Hkv + kvh) * kPage + (t % kPage)) * D) * 4 + pc * 16;
                kr[i] = *reinterpret_cast<const uint4*>(kbase + off);
                vr[i] = *reinterpret_cast<const uint4*>(vbase + off);
            } else {
                kr[i] = make_uint4(0, 0, 0, 0);
                vr[i] = make_uint4(0, 0, 0, 0);
            }
        }
    };
    auto store_chunk = [&](int buf) {
#pragma unroll
        for (int i = 0; i < C::PPT; ++i) {
            const int piece = tid + i * C::NT;
            const int kc = piece / C::ROWP;
            const int pc = piece - kc * C::ROWP;
            *reinterpret_cast<uint4*>(&s_k[buf][kc * C::KS + pc * 4]) = kr[i];
            *reinterpret_cast<uint4*>(&s_v[buf][kc * C::VS + pc * 4]) = vr[i];
        }
    };

    const int n_chunks = k_end > k_begin ? (k_end - k_begin + CHUNK - 1) / CHUNK : 0;
    if (n_chunks > 0) {
        load_chunk(0);
        store_chunk(0);
    }
    __syncthreads();

    for (int c = 0; c < n_chunks; ++c) {
        const int buf = c & 1;
        if (c + 1 < n_chunks) load_chunk(c + 1);
        const float* skb = s_k[buf];
        const float* svb = s_v[buf];

        // ---- S^T = K Q^T for the chunk's 32 keys
        f32x16 sacc;
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[e] = 0.f;
        {
            const float* krow = skb + col * C::KS;
#pragma unroll
            for (int s = 0; s < NQ; ++s) sacc = mfma_f32(krow[s + hl * (D / 2)], qf[s], sacc);
        }

        // ---- online softmax (log2 domain); key of element e: 4*hl + 8*(e/4) + e%4
        const int kb = k_begin + c * CHUNK;
        const bool need_mask = kb + CHUNK - 1 > L;
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            float x = sacc[e] * a.scale_log2;
            if (need_mask) {
                const int t = kb + hl * 4 + (e >> 2) * 8 + (e & 3);
                if (t > lim) x = -INFINITY;
            }
            sacc[e] = x;
            mx = fmaxf(mx, x);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = exp2f(m_run - m_use);
        float lsum = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const float p = exp2f(sacc[e] - m_use);
            sacc[e] = p;
            lsum += p;
        }
        l_run = l_run * alpha + lsum;
        m_run = m_new;
        if (__any(alpha != 1.f)) {
#pragma unroll
            for (int i = 0; i < C::NDT; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[i][e] *= alpha;
        }

        // ---- O^T += V^T P^T
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int key = hl * 4 + (e >> 2) * 8 + (e & 3);
            const float* vrow = svb + key * C::VS;
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt) oacc[dt] = mfma_f32(vrow[dt * 32 + col], sacc[e], oacc[dt]);
        }

        if (c + 1 < n_chunks) store_chunk(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (!row_ok) return;
    const int m_loc = m - rt * C::RT;
    if (a.nsplit == 1) {
        int slot = a.perm[(size_t)b * a.W + r];
        if (slot < 0 || slot >= a.W) {
            set_status(a.status, WEDLM_DEV_BAD_PERM);
            return;
        }
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        float* o = static_cast<float*>(a.out) + (((size_t)b * a.W + slot) * a.Hq + h) * D;
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d = dt * 32 + hl * 4 + g4 * 8;
                *reinterpret_cast<float4*>(o + d) = make_float4(oacc[dt][g4 * 4 + 0] * inv, oacc[dt][g4 * 4 + 1] * inv,
                                                                oacc[dt][g4 * 4 + 2] * inv, oacc[dt][g4 * 4 + 3] * inv);
            }
    } else {
        const size_t prow = ((size_t)pid * a.nsplit + split) * C::RT + m_loc;
        float* po = a.part_o + prow * D;
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d = dt * 32 + hl * 4 + g4 * 8;
                *reinterpret_cast<float4*>(po + d) =
                    make_float4(oacc[dt][g4 * 4 + 0], oacc[dt][g4 * 4 + 1], oacc[dt][g4 * 4 + 2], oacc[dt][g4 * 4 + 3]);
            }
        if (hl == 0) a.part_ml[prow] = make_float2(m_run, l_tot);
    }
}

// Merge the split partials of every (b, g, row) by the log-sum-exp rule and
// scatter the rows to logical slot order.  A thread owns 4 consecutive d of
// one row.  It loads the (m, l) of its row's splits and its 16-byte slices of
// the fp32 partials in batches of 8 splits, all issued before any is used,
// so one memory latency covers a batch (the D/4 threads of a row read the
// same (m, l) words: one request per wave).  No LDS, no barrier.
template <typename T, int D>
__device__ __forceinline__ void combine_rows(const AttnArgs& a, int blk, int tid) {
    constexpr int D4 = D / 4;
    constexpr int RPB = 256 / D4;
    constexpr int SB = 8;                      // splits per batch
    const int lr = tid / D4;
    const int d = (tid % D4) * 4;
    const long row = (long)blk * RPB + lr;
    int pid, m_loc, rt, kvh, b;
    if (a.tail > 0) {
        // tail plan: only the sequences cut in two have partials to merge;
        // group g is the back part's work-group, which named its sequence
        const int g = (int)(row / a.RT);
        if (g >= a.tail * a.Hkv) return;
        m_loc = (int)(row - (long)g * a.RT);
        kvh = g % a.Hkv;
        b = a.tail_seq[g];
        rt = 0;
        pid = b * a.Hkv + kvh;
    } else {
        const int npid = a.B * a.Hkv * a.row_tiles;
        pid = (int)(row / a.RT);
        if (pid >= npid) return;
        m_loc = (int)(row - (long)pid * a.RT);
        rt = pid % a.row_tiles;
        const int bk = pid / a.row_tiles;
        kvh = bk % a.Hkv;
        b = bk / a.Hkv;
    }
    const int m = rt * a.RT + m_loc;
    if (m >= a.M) return;
    const size_t base = (size_t)pid * a.nsplit * a.RT + m_loc;
    const float* po = a.part_o + base * D + d;
    const size_t stride = (size_t)a.RT * D;

    float M = -INFINITY, den = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = 0; s0 < a.nsplit; s0 += SB) {
        float2 ml[SB];
        float4 v[SB];
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            const int s = s0 + j;
            if (s < a.nsplit) {
                ml[j] = a.part_ml[base + (size_t)s * a.RT];
                v[j] = *reinterpret_cast<const float4*>(po + s * stride);
            } else {
                ml[j] = make_float2(-INFINITY, 0.f);
                v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
        // a split without keys left its O unwritten (m = -inf): weigh it zero
        // by selection, whatever the workspace holds there
#pragma unroll
        for (int j = 0; j < SB; ++j)
            if (ml[j].x == -INFINITY) v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        float Mb = M;
#pragma unroll
        for (int j = 0; j < SB; ++j) Mb = fmaxf(Mb, ml[j].x);
        if (Mb == -INFINITY) continue;         // nothing visible yet
        const float c = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mb);
        den *= c;
        acc.x *= c; acc.y *= c; acc.z *= c; acc.w *= c;
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            const float w = __builtin_amdgcn_exp2f(ml[j].x - Mb);   // 0 for empty splits
            den += w * ml[j].y;
            acc.x += w * v[j].x; acc.y += w * v[j].y; acc.z += w * v[j].z; acc.w += w * v[j].w;
        }
        M = Mb;
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    const int r = m / a.G;
    const int h = kvh * a.G + m % a.G;
    const int slot = a.perm[(size_t)b * a.W + r];
    if (slot < 0 || slot >= a.W) {
        if (d == 0) set_status(a.status, WEDLM_DEV_BAD_PERM);
        return;
    }
    T* o = static_cast<T*>(a.out) + (((size_t)b * a.W + slot) * a.Hq + h) * D + d;
    if constexpr (sizeof(T) == 2) {
        uint2 pk;
        pk.x = f32_to_bf16(acc.x * inv) | ((uint32_t)f32_to_bf16(acc.y * inv) << 16);
        pk.y = f32_to_bf16(acc.z * inv) | ((uint32_t)f32_to_bf16(acc.w * inv) << 16);
        *reinterpret_cast<uint2*>(o) = pk;
    } else {
        *reinterpret_cast<float4*>(o) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void attn_combine(AttnArgs a) {
    combine_rows<T, D>(a, blockIdx.x, threadIdx.x);
}

// Back half of a fused decode step: the commit / Eq. 11 select / refill of
// every sequence (one wave each, four per work-group, first) and the
// combine's work-groups in one launch.  They touch disjoint memory: the
// combine reads the split partials and perm and writes out; the commit reads
// the vocabulary partials and rewrites the window state and ctx_len, which
// the combine does not read.
template <typename T, int D>
__global__ __launch_bounds__(256) void step_back(AttnArgs a, SelectArgs s, int n_commit_blocks) {
    const int blk = blockIdx.x;
    if (blk < n_commit_blocks) {
        const int b = blk * 4 + (int)(threadIdx.x >> 6);
        if (b < s.B) commit_seq(s, b, threadIdx.x & 63);
    } else {
        combine_rows<T, D>(a, blk - n_commit_blocks, threadIdx.x);
    }
}

template <int D>
static unsigned combine_blocks(const AttnArgs& a) {
    constexpr int RPB = 256 / (D / 4);
    const long rows = a.tail > 0 ? (long)a.tail * a.Hkv * a.RT : (long)a.B * a.Hkv * a.row_tiles * a.RT;
    return (unsigned)((rows + RPB - 1) / RPB);
}
template <typename T, int D>
static hipError_t launch_combine_t(const AttnArgs& a, hipStream_t st) {
    hipLaunchKernelGGL((attn_combine<T, D>), dim3(combine_blocks<D>(a)), dim3(256), 0, st, a);
    return hipGetLastError();
}
template <typename T, int D>
static hipError_t launch_step_back_t(const AttnArgs& a, const SelectArgs& s, hipStream_t st) {
    const int nc = (s.B + 3) / 4;
    hipLaunchKernelGGL((step_back<T, D>), dim3(combine_blocks<D>(a) + (unsigned)nc), dim3(256), 0, st, a, s, nc);
    return hipGetLastError();
}

template <int D, int NW>
static hipError_t launch_f32_t(const AttnArgs& a, hipStream_t st, const LaunchTiming* tm) {
    const int npid = a.B * a.Hkv * a.row_tiles;
    if (tm)
        hipExtLaunchKernelGGL((attn_split_f32<D, NW>), dim3((unsigned)npid * a.nsplit), dim3(64 * NW), 0, st,
                              tm->start, tm->stop, 0, a);
    else
        hipLaunchKernelGGL((attn_split_f32<D, NW>), dim3((unsigned)npid * a.nsplit), dim3(64 * NW), 0, st, a);
    return hipGetLastError();
}

int attn_chunk(int dtype, int nw) { return dtype == WEDLM_BF16 ? 64 : 32; }

hipError_t launch_attn_bf16_split(const AttnArgs& a, int D, int nrg, hipStream_t st, const LaunchTiming* tm);

hipError_t launch_attn_split(const AttnArgs& a, int dtype, int D, int nw, hipStream_t st, const LaunchTiming* tm) {
    if (dtype == WEDLM_F32) {
        if (D == 64)
            return nw == 1 ? launch_f32_t<64, 1>(a, st, tm) : nw == 2 ? launch_f32_t<64, 2>(a, st, tm)
                                                             : launch_f32_t<64, 4>(a, st, tm);
        return nw == 1 ? launch_f32_t<128, 1>(a, st, tm) : nw == 2 ? launch_f32_t<128, 2>(a, st, tm)
                                                          : launch_f32_t<128, 4>(a, st, tm);
    }
    return launch_attn_bf16_split(a, D, nw, st, tm);
}

hipError_t launch_attn(const AttnArgs& a, int dtype, int D, int nw, hipStream_t st) {
    const hipError_t e = launch_attn_split(a, dtype, D, nw, st);
    if (e != hipSuccess || a.nsplit == 1) return e;
    if (dtype == WEDLM_F32) return D == 64 ? launch_combine_t<float, 64>(a, st) : launch_combine_t<float, 128>(a, st);
    return D == 64 ? launch_combine_t<bf16_t, 64>(a, st) : launch_combine_t<bf16_t, 128>(a, st);
}

hipError_t launch_step_back(const AttnArgs& a, const SelectArgs& s, int dtype, int D, hipStream_t st) {
    if (a.nsplit == 1) return launch_commit(s, st);
    if (dtype == WEDLM_F32) return D == 64 ? launch_step_back_t<float, 64>(a, s, st) : launch_step_back_t<float, 128>(a, s, st);
    return D == 64 ? launch_step_back_t<bf16_t, 64>(a, s, st) : launch_step_back_t<bf16_t, 128>(a, s, st);
}

}  // namespace wedlm
