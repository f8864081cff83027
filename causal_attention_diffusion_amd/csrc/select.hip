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
// second launch.  The bodies live in select.hpp: the fused decode step runs
// the same code inside its own launches (reorder.hip, attn.hip).
#include "select.hpp"

namespace wedlm {

// One (row, part) unit per 256-thread work-group.
template <bool VEC>
__global__ __launch_bounds__(kVocabThreads) void vocab_stats(SelectArgs a) {
    __shared__ Stat s_red[4];
    vocab_unit<VEC>(a, blockIdx.x, true, threadIdx.x, s_red);
}

// Commit / Eq. 11 select / refill of one sequence per 64-thread work-group
// (one lane per slot), after vocab_stats has written every row partial.
__global__ __launch_bounds__(64) void commit_select_refill(SelectArgs a) {
    commit_seq(a, blockIdx.x, threadIdx.x);
}

hipError_t launch_select(const SelectArgs& a, hipStream_t st) {
    dim3 grid((unsigned)(a.B * a.W * a.nparts)), block(kVocabThreads);
    if (vocab_vec(a))
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
