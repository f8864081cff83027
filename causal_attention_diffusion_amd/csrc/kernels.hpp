// kernels.hpp -- argument blocks and launchers of the decode-step kernels
// (one struct per kernel family, passed by value as the kernel argument).
#pragma once

#include "common.hpp"

namespace wedlm {

constexpr int kMaxSplitPages = 2048;  // LDS block-table slice of a split: split_keys <= 32768

struct ReorderArgs {
    const uint8_t* filled;
    const int32_t* pos;
    const void* q;
    const void* k;
    const void* v;
    void* q_phys;
    void* k_cache;
    void* v_cache;
    const int32_t* block_table;
    const int32_t* ctx_len;
    int32_t* perm;
    int32_t* status;
    int B, W, Hq, Hkv, D, max_pages, num_pages;
    double log2_base;
    // Projection form (reorder_from_partials): q, k and v are read as the
    // bf16-rounded sums of part_S fp32 split-K partials [part_S][B*W][part_N]
    // of the stacked [Wq; Wk; Wv] projection (q columns, then k, then v).
    const float* part;
    int part_S, part_N;
};

struct AttnArgs {
    const void* q;  // q_phys [B][W][Hq][D]
    const void* k_cache;
    const void* v_cache;
    const int32_t* block_table;
    const int32_t* ctx_len;
    const int32_t* perm;
    void* out;
    float* part_o;   // [npid][nsplit][RT][D]
    float2* part_ml; // [npid][nsplit][RT]  (m in log2 units, l)
    int32_t* status;
    int B, W, Hq, Hkv, G, M, max_pages, num_pages;
    int RT, row_tiles, nsplit, split_keys;  // split_keys: largest split (host bound)
    int split_align;   // keys per ring stage of the split kernel (64 bf16, 32 fp32)
    int max_ctx;       // host bound on ctx_len: the split grid covers max_ctx + W keys
    float scale_log2;  // softmax scale * log2(e)
    // Tail splits (bf16, one row tile, nsplit == 2; 0 = off): ids [0, B*Hkv)
    // run the first split of every (sequence, KV head) -- the whole sequence
    // unless it is one of the `tail` longest, which are cut in two -- and
    // ids past them the back parts, longest sequence first.  tail_seq
    // [tail * Hkv] receives the sequence of each back part (for the
    // combine, which merges only those).
    int tail;
    int tail_free;      // CUs without a first-round work-group (back parts that start at once)
    int32_t* tail_seq;
};

// First key of the back part of a sequence with T_len keys cut in two by the
// tail plan.  The back part's work-group starts when a CU frees up: at once
// for the first tail_free of them, else when the first-round work-groups of
// a short sequence finish (start_keys: that sequence's keys, a stand-in for
// its time).  Both parts would end together at one streaming rate when the
// front part takes (T_len + start_keys) / 2 keys, rounded up to the ring
// stage, at most T_len.
__device__ __forceinline__ int tail_cut(int T_len, int start_keys, int align) {
    const int h = ((T_len + start_keys + 1) / 2 + align - 1) / align * align;
    return h < T_len ? h : T_len;
}

struct SelectArgs {
    const float* logits;
    int32_t* tok;
    uint8_t* filled;
    int32_t* pos;
    int32_t* ctx_len;
    int32_t* n_commit;
    int32_t* committed;
    int32_t* argmax_out;
    float* entropy_out;
    int64_t* counters;    // [B][2] (N_new, N_total) accumulated, or nullptr
    float4* part;         // [B*W][nparts]: (m, argmax bits, S, T)
    int B, W, V, nparts, part_len;
    float alpha, tau;
    int mask_id;
};

struct LmheadArgs {
    const bf16_t* hidden;   // [R][Dm], R = B*W rows in (b, j) order
    const bf16_t* lm_head;  // [V][Dm]
    const uint8_t* filled;  // [R]
    int32_t* rows;          // workspace [R]: global row of each masked row, in order
    int32_t* count;         // workspace: number of masked rows
    float4* part;           // workspace [R][nvt]: (m, argmax bits, S, T) per masked row and vocab tile
    float4* row_stat;       // workspace [R]: merged statistics of each masked row (by global row)
    int R, Dm, V, nvt, nrg;  // nvt vocab tiles of kLmNT; nrg row groups (set by the launcher)
};
constexpr int kLmNT = 256;  // vocabulary entries per LM-head work-group
constexpr int kLmMT = 128;  // masked rows per LM-head work-group of the small-window shape
constexpr int kLmKC = 64;   // the hidden size must be a multiple of this

// Keys per split of one sequence: its visible keys T_len spread evenly over
// the grid's nsplit work-groups, rounded up to the ring stage `align` and
// never above split_keys (the host sized split_keys * nsplit for the longest
// admissible context, so the bound only bites there).  The split kernels and
// the combine use this same rule.
__device__ __forceinline__ int split_len(int T_len, int nsplit, int split_keys, int align) {
    int sk = (T_len + nsplit - 1) / nsplit;
    sk = (sk + align - 1) / align * align;
    if (sk < align) sk = align;
    return sk < split_keys ? sk : split_keys;
}

hipError_t launch_reorder(const ReorderArgs& a, int dtype, hipStream_t stream);
// bf16 reorder whose q/k/v come from split-K partials (a.part)
hipError_t launch_reorder_from_partials(const ReorderArgs& a, hipStream_t stream);
// Optional start / stop events of one launch, taken from the dispatch itself
// (hipExtLaunchKernel): the kernel's own duration, with no marker packets
// added to the stream.
struct LaunchTiming {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};
hipError_t launch_attn(const AttnArgs& a, int dtype, int D, int nw, hipStream_t stream);
// the split kernel alone (no combine)
hipError_t launch_attn_split(const AttnArgs& a, int dtype, int D, int nw, hipStream_t stream,
                             const LaunchTiming* tm = nullptr);
int attn_chunk(int dtype, int nw);
hipError_t launch_select(const SelectArgs& a, hipStream_t stream);
struct ModelRowArgs {
    const int32_t* tok;     // embed: window token ids [M]
    const bf16_t* embed;    // embed: [n_embed][N]
    int n_embed;
    float* x_res;           // residual stream [M][N] fp32
    bf16_t* h;              // bf16 output [M][N]
    const bf16_t* g;        // RMSNorm weight [N]
    const float* P;         // split-K partials [S][M][N] (SwiGLU: N = 2F, gate then up)
    int M, N, S;
    float eps;
    int32_t* status;
};
// y = X W^T for W stacked from up to three matrices along the output
// dimension: rows [0, n1) of W0, [n1, n2) of W1, [n2, N) of W2.
struct GemmArgs {
    const bf16_t* W0;       // [n1][K]
    const bf16_t* W1;       // [n2 - n1][K] (or unused when n1 == N)
    const bf16_t* W2;       // [N - n2][K]  (or unused when n2 == N)
    int n1, n2;
    const bf16_t* X;        // [M][K]
    float* P;               // [S][M][N] partial products
    int M, N, K, S, nrg;    // nrg set by the launcher
    // SwiGLU form (act != nullptr): W0 = gate [N/2][K], W1 = up [N/2][K],
    // S == 1, more than 128 rows; the launch writes act[m][c] =
    // bf16(silu(gate . x_m) * (up . x_m)) for c < N/2 instead of partials
    bf16_t* act;
};
bool gemm_swiglu_fused(int M, int S);
int gemm_splits(int M, int N, int K);
hipError_t launch_gemm(GemmArgs a, hipStream_t stream);
hipError_t launch_embed_rmsnorm(const ModelRowArgs& a, hipStream_t stream);
hipError_t launch_add_rmsnorm(const ModelRowArgs& a, hipStream_t stream);
hipError_t launch_finish_swiglu(const ModelRowArgs& a, hipStream_t stream);
hipError_t launch_lmhead(const LmheadArgs& a, hipStream_t stream);
hipError_t launch_dual_layout(uint8_t* filled_m, int32_t* pos_m, int32_t* ctx_m, int32_t* bt_m, int32_t* pos_p,
                              int32_t* ctx_p, int32_t* bt_p, int S, int N, int b, hipStream_t stream);
// commit / Eq. 11 select / refill alone, on row partials already in a.part
hipError_t launch_commit(const SelectArgs& a, hipStream_t stream);
// Fused decode step: the reorder with the vocabulary pass, then (after the
// split kernel) the combine with the commit (the commit alone when the
// plan has one split).
hipError_t launch_step_front(const ReorderArgs& r, const SelectArgs& s, int dtype, hipStream_t stream);
hipError_t launch_step_back(const AttnArgs& a, const SelectArgs& s, int dtype, int D, hipStream_t stream);

}  // namespace wedlm
