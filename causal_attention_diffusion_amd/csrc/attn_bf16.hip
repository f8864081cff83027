// attn_bf16.hip -- bf16 windowed causal GQA attention of one WeDLM decode
// step over a paged KV cache, streamed through LDS by direct global->LDS
// loads (gfx950).
//
// Pages: "WeDLM: Reconciling Diffusion Language Models with Standard Causal
// Attention for Fast Inference", paper-summary page, "Key claims" (paper
// sec. 3.2, 4.1, 5.2: after the reordering a plain causal mask lets every
// masked slot see all observed tokens; a decode step is a causal pass of
// the window over the cached prefix) and risewithvishwas WeDLM page,
// "Attention Mechanism" (lower-triangular mask).
//
// What differs from the fp32 kernel (attn.hip) is how K/V reach LDS:
//  * global_load_lds_dwordx4 writes each wave's 16-byte loads straight into
//    LDS (1 KB per wave instruction), so no VGPRs hold data in flight; rings
//    of 64-key stages keep AHEAD stages (96 KB at D = 128) in flight per
//    work-group;
//  * completion is tracked per wave with s_waitcnt vmcnt(n) and made visible
//    to the other waves by one s_barrier per chunk;
//  * LDS rows are unpadded; 16-byte chunks are XOR-swizzled per key (the
//    lane that fills LDS slot (key, c) loads global chunk c ^ f(key)), so
//    the K reads (ds_read_b128, 16 keys per 16 lanes) and the V transpose
//    reads (ds_read_b64_tr_b16, 4 keys x 4 chunks per 32 lanes) spread
//    over all banks.
// Work split: 8 waves = NRG row groups (32 query rows each) x NKG key
// groups.  The key group of a wave owns every NKG-th 32-key tile and keeps
// its own online-softmax state; the key groups are merged through LDS at
// the end, then the work-group writes either the final rows (one split)
// or a split partial for attn_combine.
#include "kernels.hpp"

namespace wedlm {

template <int D>
struct Bf16Cfg {
    static constexpr int NWAVES = 8;
    static constexpr int NT = 64 * NWAVES;
    static constexpr int SK = 64;                    // keys per stage
    static constexpr int RC = D * 2 / 16;            // 16-byte chunks per key row (8 or 16)
    // DMA runs AHEAD stages in front of the stage being computed.  K of
    // stage st is last read in iteration st, V in iteration st+1 (its PV
    // trails by one), so the K ring has AHEAD+1 slots and the V ring AHEAD+2:
    // 144 KB at D = 128 (3 stages = 96 KB in flight), 136 KB at D = 64.
    static constexpr int AHEAD = D == 128 ? 3 : 7;
    static constexpr int NKS = AHEAD + 1;
    static constexpr int NVS = AHEAD + 2;
    static constexpr int KBYTES = SK * D * 2;        // K (or V) bytes per stage
    static constexpr int STAGE = 2 * KBYTES;         // K then V
    static constexpr int LPS = STAGE / 1024 / NWAVES; // DMA instructions per wave per stage
    static constexpr int NDT = D / 32;
    static_assert(LPS * 1024 * NWAVES == STAGE, "stage must split into whole wave loads");
};

constexpr float kLazy = 8.0f;    // log2 of the largest unnormalised P
constexpr float kLazyP = 256.0f; // 2^kLazy
// cache policy of the K/V loads: non-temporal (every byte is read once per
// launch; measured 7 % faster streaming than the default policy)
constexpr int kNT = 2;

__device__ __forceinline__ int swz_k(int key, int c, int rc) { return c ^ (key & (rc - 1)); }
__device__ __forceinline__ int swz_v(int key, int c, int rc) { return c ^ ((4 * (key & 3)) & (rc - 1)); }

// s_waitcnt vmcnt(n), other counters untouched (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
__device__ __forceinline__ void block_sync() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Wait until at most `ahead` stages (LPS loads each) of this wave's DMA are
// still in flight, i.e. the stage issued `ahead` stages before the last one
// has landed.  `ahead` is clamped to MAXA (stricter waits stay correct).
template <int LPS, int MAXA>
__device__ __forceinline__ void wait_stage(int ahead) {
    static_assert(MAXA <= 7 && 7 * LPS < 64, "vmcnt range");
    if (ahead > MAXA) ahead = MAXA;
    switch (ahead) {
        case 7: wait_vm<(7 * LPS) & 63>(); break;
        case 6: wait_vm<(6 * LPS) & 63>(); break;
        case 5: wait_vm<(5 * LPS) & 63>(); break;
        case 4: wait_vm<4 * LPS>(); break;
        case 3: wait_vm<3 * LPS>(); break;
        case 2: wait_vm<2 * LPS>(); break;
        case 1: wait_vm<LPS>(); break;
        default: wait_vm<0>(); break;
    }
}

// Transpose reads of V for one 32-key tile, all d-tiles, both 16-key
// k-steps: rows key0 and key0 + 8 (k-step 0), key0 + 16 and key0 + 24
// (k-step 1) of each d-tile address; r[kk * 2 NDT + half * NDT + dt].
// Issued from inline asm with their own lgkmcnt wait: the compiler's wait
// insertion would otherwise put an s_waitcnt vmcnt(0) in front of every
// ds_read_b64_tr_b16 (it cannot tell them apart from the in-flight DMA
// writes of later stages), which would drain the prefetch ring.
template <int ROWB>
__device__ __forceinline__ void tr_tile4(const uint32_t (&ad)[4], s16x4 (&r)[16]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %16\n\t"
        "ds_read_b64_tr_b16 %1, %17\n\t"
        "ds_read_b64_tr_b16 %2, %18\n\t"
        "ds_read_b64_tr_b16 %3, %19\n\t"
        "ds_read_b64_tr_b16 %4, %16 offset:%20\n\t"
        "ds_read_b64_tr_b16 %5, %17 offset:%20\n\t"
        "ds_read_b64_tr_b16 %6, %18 offset:%20\n\t"
        "ds_read_b64_tr_b16 %7, %19 offset:%20\n\t"
        "ds_read_b64_tr_b16 %8, %16 offset:%21\n\t"
        "ds_read_b64_tr_b16 %9, %17 offset:%21\n\t"
        "ds_read_b64_tr_b16 %10, %18 offset:%21\n\t"
        "ds_read_b64_tr_b16 %11, %19 offset:%21\n\t"
        "ds_read_b64_tr_b16 %12, %16 offset:%22\n\t"
        "ds_read_b64_tr_b16 %13, %17 offset:%22\n\t"
        "ds_read_b64_tr_b16 %14, %18 offset:%22\n\t"
        "ds_read_b64_tr_b16 %15, %19 offset:%22\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]),
          "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]),
          "=&v"(r[15])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "i"(8 * ROWB), "i"(16 * ROWB), "i"(24 * ROWB));
}
// The K fragments of one tile (8 ds_read_b128, D = 128) and the V
// transpose reads of the previous tile (16 ds_read_b64_tr_b16) issued as one
// batch: the asm returns once the K reads have landed (LDS reads of a wave
// complete in order, so "at most 8 outstanding" after the first 8 V reads
// means all K are in), with the V reads still in flight while the QK MFMAs
// run; tr_wait16 waits for them before the PV MFMAs.  The V registers are
// outputs here and read-write operands of tr_wait16, and nothing between the
// two touches them (the compiler sees them as live values); no other LDS
// read is issued in between, so the counts are exact.
__device__ __forceinline__ void kv_issue(const uint32_t (&ka)[8], bf16x8 (&k)[8], const uint32_t (&ad)[4],
                                         s16x4 (&r)[16]) {
    asm volatile(
        "ds_read_b128 %0, %24\n\t"
        "ds_read_b128 %1, %25\n\t"
        "ds_read_b128 %2, %26\n\t"
        "ds_read_b128 %3, %27\n\t"
        "ds_read_b128 %4, %28\n\t"
        "ds_read_b128 %5, %29\n\t"
        "ds_read_b128 %6, %30\n\t"
        "ds_read_b128 %7, %31\n\t"
        "ds_read_b64_tr_b16 %8, %32\n\t"
        "ds_read_b64_tr_b16 %9, %33\n\t"
        "ds_read_b64_tr_b16 %10, %34\n\t"
        "ds_read_b64_tr_b16 %11, %35\n\t"
        "ds_read_b64_tr_b16 %12, %32 offset:2048\n\t"
        "ds_read_b64_tr_b16 %13, %33 offset:2048\n\t"
        "ds_read_b64_tr_b16 %14, %34 offset:2048\n\t"
        "ds_read_b64_tr_b16 %15, %35 offset:2048\n\t"
        "s_waitcnt lgkmcnt(8)\n\t"
        "ds_read_b64_tr_b16 %16, %32 offset:4096\n\t"
        "ds_read_b64_tr_b16 %17, %33 offset:4096\n\t"
        "ds_read_b64_tr_b16 %18, %34 offset:4096\n\t"
        "ds_read_b64_tr_b16 %19, %35 offset:4096\n\t"
        "ds_read_b64_tr_b16 %20, %32 offset:6144\n\t"
        "ds_read_b64_tr_b16 %21, %33 offset:6144\n\t"
        "ds_read_b64_tr_b16 %22, %34 offset:6144\n\t"
        "ds_read_b64_tr_b16 %23, %35 offset:6144"
        : "=&v"(k[0]), "=&v"(k[1]), "=&v"(k[2]), "=&v"(k[3]), "=&v"(k[4]), "=&v"(k[5]), "=&v"(k[6]), "=&v"(k[7]),
          "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]),
          "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]),
          "=&v"(r[15])
        : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "v"(ka[4]), "v"(ka[5]), "v"(ka[6]), "v"(ka[7]),
          "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]));
}
__device__ __forceinline__ void tr_wait16(s16x4 (&r)[16]) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]), "+v"(r[6]), "+v"(r[7]),
                   "+v"(r[8]), "+v"(r[9]), "+v"(r[10]), "+v"(r[11]), "+v"(r[12]), "+v"(r[13]), "+v"(r[14]),
                   "+v"(r[15]));
}
template <int ROWB>
__device__ __forceinline__ void tr_tile2(const uint32_t (&ad)[2], s16x4 (&r)[8]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %9\n\t"
        "ds_read_b64_tr_b16 %2, %8 offset:%10\n\t"
        "ds_read_b64_tr_b16 %3, %9 offset:%10\n\t"
        "ds_read_b64_tr_b16 %4, %8 offset:%11\n\t"
        "ds_read_b64_tr_b16 %5, %9 offset:%11\n\t"
        "ds_read_b64_tr_b16 %6, %8 offset:%12\n\t"
        "ds_read_b64_tr_b16 %7, %9 offset:%12\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(ad[0]), "v"(ad[1]), "i"(8 * ROWB), "i"(16 * ROWB), "i"(24 * ROWB));
}

// Value of lane l ^ 32 (v_permlane32_swap: the upper half of the first
// operand trades places with the lower half of the second).
__device__ __forceinline__ float other_half(float x, int hl) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(hl ? r[0] : r[1]);
}

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
    return (uint32_t)reinterpret_cast<uintptr_t>(p);  // low 32 bits of a shared-aperture address
}

template <int D, int NRG>
__global__ __launch_bounds__(512) void attn_split_bf16(AttnArgs a) {
    using C = Bf16Cfg<D>;
    constexpr int NKG = C::NWAVES / NRG;
    constexpr int RT = 32 * NRG;
    constexpr int MSTRIDE = D + 4;                              // merge rows, floats
    constexpr int RING = (C::NKS + C::NVS) * C::KBYTES;  // K ring, then V ring
    constexpr int MERGE = NKG * RT * MSTRIDE * 4;
    constexpr int SMEM = RING > MERGE ? RING : MERGE;
    __shared__ __attribute__((aligned(1024))) char s_ring[SMEM];
    __shared__ float2 s_ml[NKG][RT];
    __shared__ int s_pages[kMaxSplitPages];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar branches below
    const int rg = w % NRG;          // row group
    const int kg = w / NRG;          // key group
    const int hl = lane >> 5;
    const int col = lane & 31;

    // split-major order: every (sequence, KV head, row tile) gets its first
    // split dispatched before any second split, so the dispatcher hands the
    // remaining (equal-size) splits of long sequences to whichever CU frees
    // up first.  With several row tiles (W x G > 128 query rows) the row
    // tiles of one (sequence, KV head, split) stream the same K/V: they take
    // work-group ids 8 apart, which the dispatcher hands to the same XCD one
    // after the other, so the later tiles read that K/V from the XCD's L2
    // (the grid is padded to whole groups of 8; the padding returns at once).
    // Inside a split, sequences take ids from the last to the first: where a
    // batch lists its windows by increasing length (the Dual-Stream layout
    // lists each sequence's windows so), the longest are dispatched first
    // and the short ones fill the tail.
    const int nbk = a.B * a.Hkv;
    int split, bk, rt;
    bool cut = false;   // tail plan: this (sequence, KV head) is cut in two ...
    int tail_h = 0;     // ... at this key
    if (a.tail > 0) {
        // tail plan: rank the sequences by visible keys (longest first, ties
        // by index) from ctx_len, staged in the block-table slice's LDS
        __shared__ int s_tail_b, s_tail_cut, s_tail_rank;
        int* s_T = s_pages;              // [B] keys of each sequence
        int* s_byrank = s_pages + a.B;   // [B] keys of the sequence of each rank
        const int gid = (int)blockIdx.x;
        const bool second = gid >= nbk;
        const int e = second ? (gid - nbk) / a.Hkv : 0;
        const int my_b = second ? -1 : (nbk - 1 - gid) / a.Hkv;
        for (int i = tid; i < a.B; i += C::NT) {
            const int Li = a.ctx_len[i];
            const bool ok = Li >= 0 && Li <= a.max_ctx && (int64_t)Li + a.W <= (int64_t)a.max_pages * kPage;
            s_T[i] = ok ? Li + a.W : 0;
        }
        __syncthreads();
        for (int i = tid; i < a.B; i += C::NT) {
            const int Ti = s_T[i];
            int rank = 0;
            for (int j = 0; j < a.B; ++j) {
                const int Tj = s_T[j];
                rank += (Tj > Ti) | ((Tj == Ti) & (j < i));
            }
            s_byrank[rank] = Ti;
            if (i == my_b) {
                s_tail_cut = rank < a.tail;
                s_tail_rank = rank;
            }
            if (second && rank == e) s_tail_b = i;
        }
        __syncthreads();
        const int tb = second ? s_tail_b : my_b;
        const int kv = second ? (gid - nbk) % a.Hkv : (nbk - 1 - gid) % a.Hkv;
        split = second ? 1 : 0;
        cut = second || s_tail_cut;
        bk = tb * a.Hkv + kv;
        if (cut) {
            // back part j = rank * Hkv + head starts at once (j < tail_free)
            // or after the first round of the (j - tail_free) / Hkv-th
            // shortest sequence
            const int j = (second ? e : s_tail_rank) * a.Hkv + kv;
            const int start = j < a.tail_free ? 0 : s_byrank[a.B - 1 - min((j - a.tail_free) / a.Hkv, a.B - 1)];
            const int Tb = s_T[tb];
            tail_h = tail_cut(Tb, start, a.split_align);
        }
        rt = 0;
        if (second && tid == 0) a.tail_seq[gid - nbk] = tb;
        __syncthreads();   // s_T (s_pages) read by all before the block-table slice lands there
        bk = nbk - 1 - bk;  // undone by the common reversal below
    } else if (a.row_tiles == 1) {
        split = blockIdx.x / nbk;
        bk = blockIdx.x - split * nbk;
        rt = 0;
    } else {
        const int j = blockIdx.x >> 3;
        rt = j % a.row_tiles;
        const int q = (j / a.row_tiles) * 8 + (blockIdx.x & 7);
        split = q / nbk;
        bk = q - split * nbk;
        if (split >= a.nsplit) return;
    }
    bk = nbk - 1 - bk;
    const int pid = bk * a.row_tiles + rt;
    const int kvh = bk % a.Hkv;
    const int b = bk / a.Hkv;

    int L = a.ctx_len[b];
    const bool ctx_ok = L >= 0 && L <= a.max_ctx && (int64_t)L + a.W <= (int64_t)a.max_pages * kPage;
    if (!ctx_ok) {
        if (tid == 0 && split == 0 && rt == 0 && kvh == 0) set_status(a.status, WEDLM_DEV_BAD_CTX);
        L = 0;
    }
    const int T_len = ctx_ok ? L + a.W : 0;
    int k_begin, k_end;
    if (a.tail > 0) {
        const int h = cut ? min(tail_h, T_len) : T_len;
        k_begin = split == 0 ? 0 : h;
        k_end = split == 0 ? h : T_len;
    } else {
        const int sk = split_len(T_len, a.nsplit, a.split_keys, a.split_align);
        k_begin = split * sk;
        k_end = min(T_len, k_begin + sk);
    }
    // one split covers the sequence: the rows are written out directly
    const bool direct = a.nsplit == 1 || (a.tail > 0 && !cut);
    if (k_begin >= k_end && !direct) {
        // no key here: the split's rows get an empty partial (m = -inf, l = 0),
        // which attn_combine weighs zero without reading its O
        const size_t prow0 = ((size_t)pid * a.nsplit + split) * RT;
        for (int i = tid; i < RT; i += C::NT)
            if (rt * RT + i < a.M) a.part_ml[prow0 + i] = make_float2(-INFINITY, 0.f);
        return;
    }

    const int p0 = k_begin / kPage;
    const int np = k_end > k_begin ? (k_end + kPage - 1) / kPage - p0 : 0;
    for (int i = tid; i < np; i += C::NT) {
        int pg = a.block_table[(size_t)b * a.max_pages + p0 + i];
        if (pg < 0 || pg >= a.num_pages) {
            set_status(a.status, WEDLM_DEV_BAD_PAGE);
            pg = 0;  // stay in bounds; the sequence's result is meaningless and flagged
        }
        s_pages[i] = pg;
    }

    // this lane's query row
    const int m = rt * RT + rg * 32 + col;
    const bool row_ok = m < a.M;
    const int r = row_ok ? m / a.G : a.W;
    const int h = kvh * a.G + (row_ok ? m % a.G : 0);
    const int lim = L + r;
    bf16x8 qf[D / 16];
    {
        const size_t q_off = (((size_t)b * a.W + (row_ok ? r : 0)) * a.Hq + h) * D;
        const uint4* qp = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + q_off);
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
            // the stored bf16 query as it is: q . k is accumulated exactly
            // in fp32 and scaled (softmax scale * log2 e) in fp32 at the exp
            const uint4 v = row_ok ? qp[s * 2 + hl] : make_uint4(0, 0, 0, 0);
            qf[s] = __builtin_bit_cast(bf16x8, v);
        }
    }
    f32x16 oacc[C::NDT];
#pragma unroll
    for (int i = 0; i < C::NDT; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[i][e] = 0.f;
    // Softmax state of this lane's row: the reference m_ref (log2 units),
    // whether the row has seen a visible key yet, and the running sum l_run.
    const float sl2 = a.scale_log2;
    float m_ref = 0.f, l_run = 0.f;
    bool started = false;

    __syncthreads();  // s_pages visible; Q loads may still be in flight (waited below)
    wait_vm<0>();     // the Q loads count in vmcnt: retire them before the ring accounting starts

    const int n_stages = k_end > k_begin ? (k_end - k_begin + C::SK - 1) / C::SK : 0;
    const char* kbase = static_cast<const char*>(a.k_cache);
    const char* vbase = static_cast<const char*>(a.v_cache);
    const int last_key = k_end - 1;

    // DMA plan.  A stage is 4 pages of K and 4 pages of V (64 keys, one
    // (page, head) block each).  Wave w loads one whole block per stage:
    // waves 0..3 the K pages into K slot st % NKS, waves 4..7 the V pages
    // into V slot st % NVS.
    // The lane offsets inside a block (row,
    // swizzled chunk) never change, so a stage costs one page-table read per
    // wave and LPS loads with a uniform base.
    constexpr int ROWB = D * 2;
    constexpr int KPB = 1024 / ROWB;                 // keys per 1 KB block
    const bool wv_v = w >= 4;
    const int wpage = w & 3;
    const char* wbase = wv_v ? vbase : kbase;
    uint32_t lane_off[C::LPS];
    int lane_kin[C::LPS];
#pragma unroll
    for (int n = 0; n < C::LPS; ++n) {
        const int kin = n * KPB + lane / (ROWB / 16);
        const int cs = lane % (ROWB / 16);
        const int c = wv_v ? swz_v(kin, cs, C::RC) : swz_k(kin, cs, C::RC);
        lane_kin[n] = kin;
        lane_off[n] = (uint32_t)(kin * ROWB + c * 16);
    }
    static_assert(C::LPS * KPB == kPage, "one wave loads exactly one page block per stage");
    auto kslot = [&](int st) { return s_ring + (st % C::NKS) * C::KBYTES; };
    auto vslot = [&](int st) { return s_ring + (C::NKS + st % C::NVS) * C::KBYTES; };
    auto issue = [&](int st) {
        char* dst = (wv_v ? vslot(st) : kslot(st)) + wpage * C::LPS * 1024;
        const int kp = k_begin + st * C::SK + wpage * kPage;    // first key of this wave's page
        if (kp + kPage - 1 <= last_key) {
            const int pg = __builtin_amdgcn_readfirstlane(s_pages[kp / kPage - p0]);  // wave-uniform
            const char* pbase = wbase + ((size_t)pg * a.Hkv + kvh) * (kPage * ROWB);
#pragma unroll
            for (int n = 0; n < C::LPS; ++n)
                __builtin_amdgcn_global_load_lds(
                    (const void*)(pbase + lane_off[n]),
                    (__attribute__((address_space(3))) void*)(reinterpret_cast<uintptr_t>(dst + n * 1024)), 16, 0, kNT);
        } else {
            // The sequence ends inside (or before) this page.  Every row of
            // the block comes from one page: this one, or the page of the
            // last key when the block lies wholly past it.  Rows past the
            // last key reload the last key's row (finite data, masked later).
            const int kq = kp <= last_key ? kp : (last_key & ~(kPage - 1));
            const int rmax = last_key - kq;                        // last valid row in the page
            const int pg = __builtin_amdgcn_readfirstlane(s_pages[kq / kPage - p0]);
            const char* pbase = wbase + ((size_t)pg * a.Hkv + kvh) * (kPage * ROWB);
#pragma unroll
            for (int n = 0; n < C::LPS; ++n) {
                const int row = lane_kin[n] <= rmax ? lane_kin[n] : rmax;
                const uint32_t off = (uint32_t)(row * ROWB) + (lane_off[n] % ROWB);
                __builtin_amdgcn_global_load_lds(
                    (const void*)(pbase + off),
                    (__attribute__((address_space(3))) void*)(reinterpret_cast<uintptr_t>(dst + n * 1024)), 16, 0, kNT);
            }
        }
    };

    // A wave owns one 32-key tile (tt_w) of every PER-th stage.  S^T of the
    // tile of stage st is computed in iteration st together with its
    // softmax; its PV trails by one iteration, so V of stage st-1 must still
    // be resident in iteration st (the V ring has one slot more than the K
    // ring).
    constexpr int PER = NKG / 2;           // stages between two tiles of one wave (1, 2, 4)
    const int tt_w = kg % 2;               // this wave's tile inside its stages
    const int ph = kg / 2;                 // ... and which stages: st % PER == ph

    // Per-lane V transpose-read addresses inside a V slot: the 16-lane groups
    // read rows key0 = hl*4 + (lane&15)/4 (+ k-step rows, immediates) at
    // d = dt*32 + 16*((lane>>4)&1) + 4*(lane&3); the swizzle depends on
    // key & 3 only, which the immediates and the tile offset do not change.
    const int vkey = hl * 4 + ((lane & 15) >> 2);
    uint32_t vcol[C::NDT];
#pragma unroll
    for (int dt = 0; dt < C::NDT; ++dt) {
        const int d = dt * 32 + ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
        vcol[dt] = (uint32_t)(tt_w * 32 * ROWB + vkey * ROWB + swz_v(vkey, d / 8, C::RC) * 16 + (d % 8) * 2);
    }

    // V^T fragments of this wave's tile of stage st, both k-steps
    s16x4 vt[4 * C::NDT];
    auto pv_load = [&](int st) {
        const uint32_t vb = lds_u32(vslot(st));
        uint32_t va[C::NDT];
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt) va[dt] = vb + vcol[dt];
        if constexpr (C::NDT == 4) tr_tile4<ROWB>(va, vt);
        else tr_tile2<ROWB>(va, vt);
    };
    // O^T += V^T P^T with the loaded fragments and the P of that tile
    auto pv_mfma = [&](const bf16x8 (&p)[2]) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int dt = 0; dt < C::NDT; ++dt) {
                const s16x4 lo = vt[kk * 2 * C::NDT + dt], hi = vt[kk * 2 * C::NDT + C::NDT + dt];
                const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, p[kk], oacc[dt], 0, 0, 0);
            }
    };

    // S^T = K Q^T for this wave's tile of stage st, causal mask applied
    auto qk_mfma = [&](const bf16x8 (&kf)[D / 16], f32x16& sacc) {
        f32x16 zero;
#pragma unroll
        for (int e = 0; e < 16; ++e) zero[e] = 0.f;
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[0], qf[0], zero, 0, 0, 0);
#pragma unroll
        for (int s = 1; s < D / 16; ++s) sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[s], sacc, 0, 0, 0);
    };
    auto mask_tile = [&](int st, f32x16& sacc) {
        const int tb = k_begin + st * C::SK + tt_w * 32;   // first key of the tile
        if (tb + 31 > L) {        // uniform: only tiles reaching past the cached prefix
            asm volatile("");     // keep this a branch (no speculation into every tile)
            const int thr = lim - tb - hl * 4;
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if ((e >> 2) * 8 + (e & 3) > thr) sacc[e] = -INFINITY;
        }
    };
    auto qk = [&](int st, f32x16& sacc) {
        const int key = tt_w * 32 + col;
        const char* krow = kslot(st) + key * ROWB;
        bf16x8 kf[D / 16];
#pragma unroll
        for (int s = 0; s < D / 16; ++s) kf[s] = *reinterpret_cast<const bf16x8*>(krow + swz_k(key, 2 * s + hl, C::RC) * 16);
        qk_mfma(kf, sacc);
        mask_tile(st, sacc);
    };
    // The same with the V reads of stage st - 1 in flight beside it (D = 128,
    // one tile per wave and stage): kv_issue, then tr_wait16 before the PV.
    uint32_t koff[D / 16];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        const int key = tt_w * 32 + col;
        koff[s] = (uint32_t)(key * ROWB + swz_k(key, 2 * s + hl, C::RC) * 16);
    }
    auto qk_v = [&](int st, f32x16& sacc) {
        if constexpr (C::NDT == 4) {
            const uint32_t kb = lds_u32(kslot(st)), vb = lds_u32(vslot(st - 1));
            uint32_t ka[8], va[4];
#pragma unroll
            for (int s = 0; s < 8; ++s) ka[s] = kb + koff[s];
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) va[dt] = vb + vcol[dt];
            bf16x8 kf[8];
            kv_issue(ka, kf, va, vt);
            qk_mfma(kf, sacc);
            mask_tile(st, sacc);
        }
    };

    // Online softmax in the log2 domain with a lazily moved reference.  The
    // accumulator holds q . k, so P = 2^(q . k * scale log2 e - m_ref) is one
    // FMA and one v_exp per score (sm_core, branch-free: it is interleaved
    // with MFMAs).
    // The reference only has to keep P in range: sm_finish moves it when a
    // row has not seen a visible key yet or when this lane's 16 P sum past
    // 2^kLazy (so every P <= 2^kLazy holds, as with a max test; inf and NaN
    // sums also fail the test).  Then it takes the true tile maximum, moves
    // m_ref up to it when it exceeds m_ref by more than kLazy, rescales O and
    // l (O must already hold every PV before this tile's) and recomputes P.
    // The row sum adds the bf16-rounded P that the PV contraction uses.
    auto p_sum = [&](const bf16x8 (&pn)[2]) {
        const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
        float ls = 0.f;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pn[kk], pn[kk], 0, 1), ones, ls, false);
            ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pn[kk], pn[kk], 2, 3), ones, ls, false);
            ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pn[kk], pn[kk], 4, 5), ones, ls, false);
            ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pn[kk], pn[kk], 6, 7), ones, ls, false);
        }
        return ls;
    };
    auto sm_core = [&](const f32x16& sacc, bf16x8 (&pn)[2], float& lsum, bool& need) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int e = 0; e < 8; ++e) pn[kk][e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sacc[kk * 8 + e], sl2, -m_ref));
        lsum = p_sum(pn);
        need = !started || !(lsum <= kLazyP);
    };
    auto sm_finish = [&](const f32x16& sacc, bf16x8 (&pn)[2], float& lsum, bool need) {
        if (__any(need)) {
            float mx = sacc[0];
#pragma unroll
            for (int e = 1; e < 16; ++e) mx = fmaxf(mx, sacc[e]);
            mx = fmaxf(mx, other_half(mx, hl)) * sl2;                // true tile maximum (log2 units)
            const bool vis = mx != -INFINITY;
            const float m_new = started ? (mx > m_ref + kLazy ? mx : m_ref) : (vis ? mx : m_ref);
            if (__any(m_new != m_ref)) {
                // rows that had not started hold O = 0 and l = 0
                const float alpha = (started && m_new != m_ref) ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
                l_run *= alpha;
#pragma unroll
                for (int i = 0; i < C::NDT; ++i)
#pragma unroll
                    for (int e = 0; e < 16; ++e) oacc[i][e] *= alpha;
            }
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    pn[kk][e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sacc[kk * 8 + e], sl2, -m_new));
            lsum = p_sum(pn);
            m_ref = m_new;
            started = started || vis;
        }
        l_run += lsum;
    };

    // Ring step of stage st: this wave's loads of stage st landed (issued
    // stages end at min(st+AHEAD-1, n_stages-1)); the barrier makes every
    // wave's part visible and frees K slot (st-1) and V slot (st-2), whose
    // last readers ran in iteration st-1, for the DMA of stage st+AHEAD.
    auto ring_step = [&](int st) {
        if (st < n_stages) wait_stage<C::LPS, C::AHEAD - 1>(min(C::AHEAD - 1, n_stages - 1 - st));
        block_sync();
        if (st + C::AHEAD < n_stages) issue(st + C::AHEAD);
    };
    const int npro = n_stages < C::AHEAD ? n_stages : C::AHEAD;
    for (int st = 0; st < npro; ++st) issue(st);
    f32x16 sacc;
    bf16x8 pprev[2];
    if constexpr (PER == 1) {
        // Every wave has a tile in every stage.  Iteration st: QK of st (at
        // D = 128 with the V reads of st-1 in flight); then the 2*NDT PV
        // MFMAs of st-1 interleaved with the softmax VALU work of st in one
        // straight-line region, so each MFMA's pipe time covers a share of
        // the softmax.
        for (int st = 0; st < n_stages; ++st) {
            ring_step(st);
            if constexpr (C::NDT == 4) {
                if (st > 0) qk_v(st, sacc);
                else qk(st, sacc);
            } else {
                qk(st, sacc);
            }
            bf16x8 pn[2];
            float lsum;
            bool need;
            if (st > 0) {
                if constexpr (C::NDT == 4) tr_wait16(vt);
                else pv_load(st - 1);
                pv_mfma(pprev);
                sm_core(sacc, pn, lsum, need);
#pragma unroll
                for (int i = 0; i < 2 * C::NDT; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 32 / C::NDT, 0);    // then VALU
                }
                // keep P and its sum inside this region (the compiler would
                // otherwise sink them below the rescale branch)
                asm volatile("" ::"v"(pn[0]), "v"(pn[1]), "v"(lsum));
            } else {
                sm_core(sacc, pn, lsum, need);
            }
            sm_finish(sacc, pn, lsum, need);
            pprev[0] = pn[0];
            pprev[1] = pn[1];
        }
        if (n_stages > 0) {
            pv_load(n_stages - 1);
            pv_mfma(pprev);
        }
    } else {
        for (int st = 0; st <= n_stages; ++st) {
            ring_step(st);
            const bool cur = st < n_stages && (st % PER) == ph;
            const bool prev = st >= 1 && ((st - 1) % PER) == ph;
            if (cur) qk(st, sacc);
            if (prev) {
                pv_load(st - 1);
                pv_mfma(pprev);
            }
            if (cur) {
                bf16x8 pn[2];
                float lsum;
                bool need;
                sm_core(sacc, pn, lsum, need);
                sm_finish(sacc, pn, lsum, need);
                pprev[0] = pn[0];
                pprev[1] = pn[1];
            }
        }
    }

    // ---- merge the key groups through LDS
    const float l_tot = l_run + other_half(l_run, hl);
    wait_vm<0>();
    wait_lgkm0();
    block_sync();   // ring no longer read by anyone
    float* mg = reinterpret_cast<float*>(s_ring);
    {
        const int row = rg * 32 + col;
        float* dst = mg + ((size_t)kg * RT + row) * MSTRIDE;
#pragma unroll
        for (int dt = 0; dt < C::NDT; ++dt)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4)
                *reinterpret_cast<float4*>(dst + dt * 32 + hl * 4 + g4 * 8) =
                    make_float4(oacc[dt][g4 * 4 + 0], oacc[dt][g4 * 4 + 1], oacc[dt][g4 * 4 + 2], oacc[dt][g4 * 4 + 3]);
        if (hl == 0) s_ml[kg][row] = make_float2(started ? m_ref : -INFINITY, l_tot);
    }
    __syncthreads();

    constexpr int D4 = D / 4;
    for (int idx = tid; idx < RT * D4; idx += C::NT) {
        const int row = idx / D4;
        const int d = (idx % D4) * 4;
        const int mm = rt * RT + row;
        if (mm >= a.M) continue;
        float M = -INFINITY;
#pragma unroll
        for (int g = 0; g < NKG; ++g) M = fmaxf(M, s_ml[g][row].x);
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
        float Ls = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int g = 0; g < NKG; ++g) {
                const float2 ml = s_ml[g][row];
                const float wgt = __builtin_amdgcn_exp2f(ml.x - M);
                Ls += wgt * ml.y;
                const float4 v = *reinterpret_cast<const float4*>(mg + ((size_t)g * RT + row) * MSTRIDE + d);
                o.x += wgt * v.x; o.y += wgt * v.y; o.z += wgt * v.z; o.w += wgt * v.w;
            }
        }
        if (direct) {
            const int rr = mm / a.G;
            const int hh = kvh * a.G + mm % a.G;
            const int slot = a.perm[(size_t)b * a.W + rr];
            if (slot < 0 || slot >= a.W) {
                set_status(a.status, WEDLM_DEV_BAD_PERM);
                continue;
            }
            const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
            uint16_t* op = static_cast<uint16_t*>(a.out) + (((size_t)b * a.W + slot) * a.Hq + hh) * D + d;
            uint2 pk;
            pk.x = f32_to_bf16(o.x * inv) | ((uint32_t)f32_to_bf16(o.y * inv) << 16);
            pk.y = f32_to_bf16(o.z * inv) | ((uint32_t)f32_to_bf16(o.w * inv) << 16);
            *reinterpret_cast<uint2*>(op) = pk;
        } else {
            const size_t prow = ((size_t)pid * a.nsplit + split) * RT + row;
            *reinterpret_cast<float4*>(a.part_o + prow * D + d) = o;
            if (d == 0) a.part_ml[prow] = make_float2(M, Ls);
        }
    }
}

// Work-groups of the split kernel: one per (sequence, KV head, row tile,
// split); with several row tiles the (sequence, KV head, split) groups are
// padded to a multiple of 8 (see the id mapping in the kernel).
static unsigned bf16_split_grid(const AttnArgs& a) {
    if (a.tail > 0) return (unsigned)((long)a.B * a.Hkv + (long)a.tail * a.Hkv);
    const long groups = (long)a.B * a.Hkv * a.nsplit;
    if (a.row_tiles == 1) return (unsigned)groups;
    return (unsigned)((groups + 7) / 8 * 8 * a.row_tiles);
}

template <int D, int NRG>
static hipError_t launch_bf16_t(const AttnArgs& a, hipStream_t st, const LaunchTiming* tm) {
    if (tm)
        hipExtLaunchKernelGGL((attn_split_bf16<D, NRG>), dim3(bf16_split_grid(a)), dim3(512), 0, st, tm->start,
                              tm->stop, 0, a);
    else
        hipLaunchKernelGGL((attn_split_bf16<D, NRG>), dim3(bf16_split_grid(a)), dim3(512), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_attn_bf16_split(const AttnArgs& a, int D, int nrg, hipStream_t st, const LaunchTiming* tm) {
    if (D == 64) {
        if (nrg == 1) return launch_bf16_t<64, 1>(a, st, tm);
        if (nrg == 2) return launch_bf16_t<64, 2>(a, st, tm);
        return launch_bf16_t<64, 4>(a, st, tm);
    }
    if (nrg == 1) return launch_bf16_t<128, 1>(a, st, tm);
    if (nrg == 2) return launch_bf16_t<128, 2>(a, st, tm);
    return launch_bf16_t<128, 4>(a, st, tm);
}

}  // namespace wedlm
