// Internal declarations of libmedusa: the per-call tree description handed
// to kernels and the launchers each kernel file exports to the dispatcher.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#define MD_WAVE 64

// A validated tree, expanded on the host and passed to kernels by value.
struct DevTree {
    int32_t n;
    int32_t max_depth;
    int8_t parent[64];
    int8_t depth[64];
    int8_t rank[64];
    // Hydra: the nodes that have children, ordered by depth then index;
    // level i (children at depth i) owns lp[level_off[i] .. level_off[i+1]).
    int8_t lp[64];
    int8_t prow[64];        // a node's position among its level's parents (-1: leaf)
    int32_t level_off[10];  // i = 1..9 used; level_off[i+1]-level_off[i] = P_i
    uint64_t anc[64];       // bit j set: node j is this node or one of its ancestors
};

// A token for one launch of a kernel whose blocks meet through flag words
// (md_sync.h): never 0, distinct across the process's launches, and started
// at a random value so that a workspace last used by another process cannot
// hold it (api.cpp).
uint64_t launch_token();

// Compute units of the current device (256 if the query fails).
inline int device_cus() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                   hipSuccess || n <= 0)
        n = 256;
    return n;
}

// ---- heads (heads.hip) ----
struct HeadsArgs {
    int kind;  // 0 Medusa, 1 Hydra (a shared projection is Medusa with shared_u)
    int shared_u;  // 1: one U [V][d] for every head
    int dt;    // 0 f32, 1 bf16
    int M;     // rows through the heads this call
    int B;     // Hydra: requests
    int d, din, V;
    int nh;     // heads this call (K or 1)
    int head0;  // first head's index in W, b, U
    int kk[8];  // top-k width per head slot
    int kmax;
    int level;
    const void* h;
    const void* W;
    const void* b;
    const void* U;
    const void* U_op;  // optional operand-order copy of U (bf16), read by the few-row matrix-core kernels
    const float* U_norms;  // optional largest squared row norm of U per 256-row tile (bf16), read by the certified pass
    const void* W_op;      // optional operand-order copy of W (bf16), read by the few-row residual kernels
    const void* E;
    const int32_t* root_tok;
    const int32_t* tree_tok;
    int32_t* topk_idx;
    float* topk_val;
    float* h_res;
    void* ws;
    float* logits;  // non-null: write every logit [M][logits_k][V] instead of the top-k (GEMV path)
    int logits_k;
    int spin_res, spin_lists;  // polls of the single-launch kernel's bounded waits (-1: the built-in limits)
};

size_t heads_ws_bytes(int dt, int M, int d, int din, int V, int nh, int kmax, int shared_u, bool op);  // this plan
size_t heads_ws_bound(int dt, int M, int d, int din, int V, int nh, int kmax, int shared_u);  // any plan of these sizes
// one Medusa row in bf16 through per-head projections: one fused launch (residual, projection, top-k, merge)
bool heads_fused_applicable(int dt, int M, int d, int din, int shared_u, int nh);
// matrix-core path for many rows (heads_mfma.hip)
bool heads_mfma_applicable(int dt, int M, int d, int din, bool op, int rows_v);  // rows_v: projection columns
// one Medusa row with an operand-order copy (shared projection): the GEMV residual feeds the matrix cores
bool residual_on_gemv(int dt, int kind, int M, int d, int din, bool op);
hipError_t residual_gemv_split(const HeadsArgs& a, const DevTree* tree, float* hres, uint16_t* hhi, uint16_t* hlo,
                               int* bound, int bound_init, hipStream_t s);
size_t heads_mfma_ws_bytes(int M, int d, int din, int V, int nh, int kmax, int shared_u);
// float32 rounding allowance of the certified pass per unit |U_v| |h'| at contraction length d
float cert_rounding_allowance(int d);
hipError_t heads_mfma_launch(const HeadsArgs& a, const DevTree* tree, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1,
                             float** part_val, int** part_idx, int* nlists);
hipError_t heads_launch(const HeadsArgs& a, const DevTree* tree, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1);
size_t heads_logits_ws_bytes(int M, int d, int nh);
// the k-way merge of nlists sorted lists per (row, head): lists [nh][M][nlists][kmax] -> [M][nh][kmax]
hipError_t topk_merge_launch(const float* pv, const int* pi, int M, int nh, int nlists, const int* kk, int kmax,
                             int32_t* idx, float* val, hipStream_t s);
bool argmax_mfma_applicable(int dt, int R, int d, bool op);
size_t argmax_mfma_ws_bytes(int R, int V);
hipError_t argmax_mfma_launch(int R, int d, int V, const void* H, const void* Wt, const void* Wt_op, void* ws,
                              hipStream_t s, float** part_val, int** part_idx, int* nlists);
// the largest squared row norm of each 256-row tile of nmat [V][d] bf16 matrices -> out [nmat][ceil(V / 256)]
hipError_t vocab_tile_norms_launch(const void* U, int nmat, int V, int d, float* out, hipStream_t s);
int vocab_tiles(int V);
// the operand-order copy of nmat row-major [rows][cols] bf16 matrices (heads_mfma.hip)
size_t operand_order_bytes(int nmat, int rows, int cols);
hipError_t operand_order_launch(int nmat, int rows, int cols, const void* src, void* dst, hipStream_t s);

// ---- the target's LM head with a fused argmax (heads.hip) ----
size_t target_argmax_ws_bound(int dt, int R, int d, int V);
hipError_t target_argmax_launch(int dt, int R, int d, int V, const void* H, const void* Wt, const void* Wt_op,
                                int32_t* tok, float* val, void* ws, hipStream_t s);

// ---- tree build (tree.hip) ----
hipError_t tree_build_launch(const DevTree& t, int kind, int B, int M, int K, int kmax, int level,
                             const int32_t* topk_idx,
                             const int32_t* src_row, const int32_t* root_tok, const int32_t* lens,
                             int32_t* tree_tok, int32_t* tree_pos, hipStream_t s);

// ---- tree attention (attention.hip) ----
struct AttnPlan {
    int splits;     // key-range splits per (request, kv head, query tile)
    int chunk;      // keys per split (multiple of the key tile)
    int qtiles;     // query tiles per (request, kv head)
    int rows;       // query rows per (request, kv head) = N * Hq / Hkv
    int rg;         // 16-row query groups per wave of the matrix-core kernel (1 or 2)
};
AttnPlan attention_plan(int dt, int B, int N, int Hq, int Hkv, int hd, int max_len);
size_t attention_ws_bytes(int dt, int B, int N, int Hq, int Hkv, int hd, int max_len);
hipError_t attention_launch(const DevTree& t, int dt, int B, int Hq, int Hkv, int hd, int Lcap, int max_len,
                            const void* q, const void* Kc, const void* Vc, const int32_t* lens, float scale,
                            void* out, void* ws, hipStream_t s);
// the library's static attention scratch of the current device (md_tree_attention_noalloc)
constexpr size_t kAttnScratchBytes = (size_t)32 << 20;
hipError_t attention_scratch(void** ptr);

// ---- accept (accept.hip) ----
size_t accept_ws_bytes(int B, int N, int V);
hipError_t accept_launch(const DevTree& t, int dt, int B, int K, int V, int Hkv, int hd, int Lcap,
                         const float* logits, const int32_t* tree_tok, void* Kc, void* Vc, int32_t* lens,
                         int32_t* accept_len, int32_t* path, int32_t* next_tok, int32_t* compact_src, void* ws,
                         hipStream_t s);
hipError_t accept_tokens_launch(const DevTree& t, int dt, int B, int K, int Hkv, int hd, int Lcap,
                                const int32_t* target_tok, const int32_t* tree_tok, void* Kc, void* Vc,
                                int32_t* lens, int32_t* accept_len, int32_t* path, int32_t* next_tok,
                                int32_t* compact_src, hipStream_t s);

// ---- sampled decoding (sample.hip) ----
size_t draft_sample_ws_bytes(int M, int K, int V, int kmax);
hipError_t draft_sample_launch(int M, int K, int V, const int* kk, int kmax, float T, const float* logits,
                               const uint32_t* words, int32_t* tok, float* lse, void* ws, hipStream_t s);
size_t verify_sampled_ws_bytes(int B, int N);
hipError_t verify_sampled_launch(const DevTree& t, int dt, int B, int K, int V, int Hkv, int hd, int Lcap, float T,
                                 const float* target_logits, const float* head_logits, const float* head_lse,
                                 const int32_t* tree_tok, const uint32_t* u_words, const uint32_t* g_words,
                                 void* Kc, void* Vc, int32_t* lens, int32_t* accept_len, int32_t* path,
                                 int32_t* next_tok, int32_t* compact_src, void* ws, hipStream_t s);
size_t accept_typical_ws_bytes(int B, int N);
hipError_t accept_typical_launch(const DevTree& t, int dt, int B, int K, int V, int Hkv, int hd, int Lcap, float T,
                                 float eps, float delta, const float* target_logits, const int32_t* tree_tok,
                                 const uint32_t* g_words, void* Kc, void* Vc, int32_t* lens, int32_t* accept_len,
                                 int32_t* path, int32_t* next_tok, int32_t* compact_src, void* ws, hipStream_t s);

// ---- measurement utility (probe.hip) ----
int probe_blocks();
hipError_t probe_launch(const void* buf, size_t bytes, void* sink, hipStream_t s);
