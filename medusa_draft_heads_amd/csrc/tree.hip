// The candidate tree's tokens and positions.
//
// "Medusa heads versus separate draft model", section "Trees": the step forms
// a tree of combinations of each head's best candidates. With a fixed
// topology, node n at depth j carries entry rank(n) of head j's list: for
// Medusa the list of the row that builds the request's tree, for Hydra
// (abstract; summary) the list its own parent's row produced. The root is the
// target's own next token. One wave per request, one lane per node.
#include "md_internal.h"

namespace {

__global__ __launch_bounds__(MD_WAVE) void k_tree_medusa(DevTree t, int M, int K, int kmax,
                                                         const int32_t* __restrict__ topk_idx,
                                                         const int32_t* __restrict__ src_row,
                                                         const int32_t* __restrict__ root_tok,
                                                         const int32_t* __restrict__ lens, int32_t* __restrict__ tok,
                                                         int32_t* __restrict__ pos) {
    const int b = blockIdx.x, n = threadIdx.x;
    if (n >= t.n) return;
    const int dep = t.depth[n];
    int v;
    if (n == 0) {
        v = root_tok[b];
    } else {
        const int row = src_row[b];
        // a source row outside [0, M) names no list: the node gets no token
        v = (row >= 0 && row < M) ? topk_idx[((int64_t)row * K + dep - 1) * kmax + t.rank[n]] : -1;
    }
    tok[(int64_t)b * t.n + n] = v;
    pos[(int64_t)b * t.n + n] = lens[b] + dep;
}

__global__ __launch_bounds__(MD_WAVE) void k_tree_hydra(DevTree t, int kmax, int level,
                                                        const int32_t* __restrict__ topk_idx,
                                                        const int32_t* __restrict__ root_tok,
                                                        const int32_t* __restrict__ lens, int32_t* __restrict__ tok,
                                                        int32_t* __restrict__ pos) {
    const int b = blockIdx.x, n = threadIdx.x;
    if (n >= t.n) return;
    const int dep = t.depth[n];
    const int P = t.level_off[level + 1] - t.level_off[level];
    if (level == 1) {
        pos[(int64_t)b * t.n + n] = lens[b] + dep;
        if (n == 0) tok[(int64_t)b * t.n] = root_tok[b];
    }
    if (dep == level) {
        const int row = b * P + t.prow[t.parent[n]];
        tok[(int64_t)b * t.n + n] = topk_idx[(int64_t)row * kmax + t.rank[n]];
    }
}

}  // namespace

hipError_t tree_build_launch(const DevTree& t, int kind, int B, int M, int K, int kmax, int level,
                             const int32_t* topk_idx, const int32_t* src_row, const int32_t* root_tok,
                             const int32_t* lens, int32_t* tree_tok, int32_t* tree_pos, hipStream_t s) {
    if (kind == 0)
        hipLaunchKernelGGL(k_tree_medusa, dim3(B), dim3(MD_WAVE), 0, s, t, M, K, kmax, topk_idx, src_row, root_tok,
                           lens, tree_tok, tree_pos);
    else
        hipLaunchKernelGGL(k_tree_hydra, dim3(B), dim3(MD_WAVE), 0, s, t, kmax, level, topk_idx, root_tok, lens,
                           tree_tok, tree_pos);
    return hipGetLastError();
}
