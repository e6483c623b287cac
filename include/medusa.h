/*
 * libmedusa -- the Medusa tree-decode step on AMD Instinct MI355X (gfx950).
 *
 * One decode step, as the pages describe it:
 *   1. md_medusa_heads  K draft heads on the target's last hidden state, each a
 *                       residual block h + SiLU(W h + b) followed by its own
 *                       d x V vocabulary projection, reduced straight to each
 *                       head's top-k (the logits never reach memory).
 *                       ("Medusa heads versus separate draft model", sections
 *                       "What each one is" and "Cost per step".) Hydra's
 *                       sequentially dependent heads run one level per call
 *                       (Hydra abstract and summary).
 *   2. md_tree_build    the candidate tree: every node takes one entry of its
 *                       head's top-k list at a fixed topology ("Trees").
 *   3. md_tree_attention every tree node attends to the KV cache and to its
 *                       own root path, all in one pass ("Trees": one pass with
 *                       a tree attention mask).
 *   4. md_tree_accept   the target's greedy choice per node, the deepest branch
 *                       whose drafts all match it, and the move of that
 *                       branch's cache entries next to the prefix ("Trees":
 *                       the step advances along the branch that matches;
 *                       "Acceptance": E counts the target's token plus the
 *                       accepted drafts).
 *
 * Conventions for every call
 *  - Pointers marked (device) are HIP device pointers; (host) are host memory.
 *    The caller owns every buffer. The library allocates and frees nothing and
 *    keeps no pointer past the call.
 *  - `stream` is a hipStream_t (NULL: the null stream). Calls only enqueue
 *    work and return; outputs are valid once the stream reaches that point.
 *    No call synchronises the host.
 *  - All argument checks run on the host before any HIP call. A non-zero
 *    return means nothing was enqueued (except MD_EHIP, which reports a
 *    failed launch). md_last_error() gives a thread-local description.
 *  - Tensors are dense row-major (C order). dt selects the storage type of
 *    activations, weights and the KV cache: MD_F32 or MD_BF16. Arithmetic is
 *    float32 throughout.
 *  - Inputs must be finite; NaN or Inf inputs give unspecified results.
 *  - Calls that overlap on one workspace race; one workspace per stream.
 */
#ifndef MEDUSA_H
#define MEDUSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MD_OK = 0,
    MD_EINVAL = -1,       /* null pointer, non-positive size, malformed tree */
    MD_EUNSUPPORTED = -2, /* a size outside what the kernels implement */
    MD_ERANGE = -3,       /* lengths that do not fit the cache capacity */
    MD_EWORKSPACE = -4,   /* workspace smaller than the *_workspace_bytes query */
    MD_EHIP = -5          /* a HIP launch or runtime call failed */
} md_status;

typedef enum { MD_F32 = 0, MD_BF16 = 1 } md_dtype;
typedef enum { MD_HEADS_MEDUSA = 0, MD_HEADS_HYDRA = 1, MD_HEADS_MEDUSA_SHARED = 2 } md_heads_kind;

#define MD_MAX_NODES 64 /* a tree fits one 64-lane wavefront and one 64-bit mask */
#define MD_MAX_HEADS 8
#define MD_MAX_TOPK 16

/* A fixed tree topology (host memory, passed by pointer, copied per call).
 * Node 0 is the root (the target's own next token). For n >= 1, parent[n] is
 * an earlier node (0 <= parent[n] < n), depths never decrease with the node
 * index (breadth-first numbering), and rank[n] is the entry of the depth-j
 * head's top-k list that node n carries (j = depth of n). Siblings carry
 * distinct ranks. parent[0] = -1, rank[0] = 0. Entries at n >= `n` are
 * ignored. */
typedef struct {
    int32_t n;
    int8_t parent[MD_MAX_NODES];
    int8_t rank[MD_MAX_NODES];
} md_tree;

/* Checks a topology against K heads with top-k widths k_per_head[K] (host):
 * 1 <= n <= 64, parent order, breadth-first numbering, depth <= K, distinct
 * sibling ranks, rank < k_per_head[depth - 1]. Host only; returns MD_OK or
 * MD_EINVAL. */
int md_tree_validate(const md_tree* t, int K, const int32_t* k_per_head);

/* Bytes of weights one call of the heads reads: K heads of (d x din residual
 * matrix + d bias + V x d projection), din = d (Medusa) or 2d (Hydra), at the
 * storage size of dt ("Cost per step": 1,117.8M parameters per head at
 * d = 8,192, V = 128,256). With one projection shared by the heads
 * (MD_HEADS_MEDUSA_SHARED) the V x d matrix counts once ("What interviewers
 * probe next": sharing saves 3.15B of the 4.47B). Returns -1 on invalid
 * arguments. */
int64_t md_heads_weight_bytes(int kind, int dt, int d, int V, int K);

/* Workspace the heads need for M rows (Medusa, shared or not) or the largest
 * level's rows (Hydra: B requests times the most parents on one level, at
 * most 64 * B), with or without an operand-order copy of U. */
size_t md_heads_workspace_bytes(int kind, int dt, int M, int d, int V, int K, int kmax);

/* 1 when md_medusa_heads runs these sizes as a single launch (one bf16 row
 * through per-head projections, kind MD_HEADS_MEDUSA): the residual blocks,
 * the vocabulary projections, the per-head top-k and their merge in one
 * kernel, so W streams in the same kernel as U and no merge kernel follows;
 * else 0. Host only. */
int md_heads_fused(int kind, int dt, int M, int d, int K);

/* Many bf16 rows (more than 128 through the projection) take a certified
 * single-product pass: the matrix cores form U.hi only, every logit is
 * known to within E = N ((1 + 2^-7) |h' - hi| + c(d) |h'|) of it (N the
 * largest row norm of U in a 256-row tile, Cauchy-Schwarz), entries that
 * cannot reach the top k are dropped and the rest re-scored from hi + lo, so
 * the lists are those of the float32 re-scored logits over the whole
 * vocabulary. This returns c(d): the float32 rounding allowance of both
 * sums per unit |U_v| |h'| at contraction length d, from the recursive
 * summation bound gamma_n = n u / (1 - n u), u = 2^-24, over d / 32 + 32
 * roundings of the matrix-core sum and d / 64 + 6 of the re-scoring. Host
 * only; -1 for d < 1. */
float md_certified_rounding_allowance(int d);

/* Operand order: a copy of nmat row-major bf16 matrices [rows][cols] laid
 * out for the matrix cores, written once when the weights load. Every MFMA
 * operand fragment (16 rows x 32 contraction elements, 1 KB) is contiguous
 * in lane order (lane l: row l % 16, elements 8 (l / 16) .. + 7), ordered
 * [tile of 256 rows][step of 32 columns][16-row block][64 lanes][8]; rows
 * past `rows` are zero. The heads and the LM head read such a copy, when
 * given one, in their few-row matrix-core kernels: one step of a 256-row
 * tile is then 16 KB of consecutive memory instead of 16 runs of 64 bytes
 * per load (the row-major reads of those kernels stream at ~4.8 TB/s on
 * MI355X, consecutive 1 KB loads at ~7). The row-major matrix stays the
 * primary input (the GEMV path and the re-scoring of the certified pass read
 * rows of it). */
/* Bytes of the copy: nmat * ceil(rows / 256) * 256 * cols * 2; 0 when
 * nmat < 1, rows < 1 or cols is not a positive multiple of 32. */
size_t md_operand_order_bytes(int nmat, int rows, int cols);
/* Writes the copy of src (device, bf16, [nmat][rows][cols]) to dst (device,
 * md_operand_order_bytes(...) bytes; caller-owned, must not overlap src).
 * Errors: MD_EINVAL (nmat or rows < 1, NULL pointers), MD_EUNSUPPORTED
 * (cols not a positive multiple of 32), MD_EHIP. */
int md_operand_order(int nmat, int rows, int cols, const void* src, void* dst, void* stream);

/* Tile norms of a vocabulary matrix, made once when the weights load.
 *
 * The many-row heads (more than 128 bf16 rows, e.g. 64 tree nodes x batch 8)
 * run one bf16 product per logit and certify the top-k against a rounding
 * allowance that scales with the largest row norm of U in each 256-row
 * vocabulary tile ("What each one is", "Trees": the k best of each head's
 * logits). Those norms depend on U alone; given this table the pass reads
 * them instead of computing them on the matrix cores at every call.
 * norms[mat][t] = max over rows v in [256 t, 256 t + 256) of the sum over
 * j of U[mat][v][j]^2 (rows past V count 0), float32, computed from the bf16
 * values (their squares are exact in float32; the sum's relative rounding
 * error stays below 2^-16 for d <= 2^14, well inside the pass's margin). */
/* Bytes of the table: nmat * ceil(V / 256) * 4; 0 when nmat or V < 1. */
size_t md_vocab_tile_norms_bytes(int nmat, int V);
/* Writes the table of U (device, bf16, [nmat][V][d]) to norms (device,
 * md_vocab_tile_norms_bytes(...) bytes, caller-owned).
 * Errors: MD_EINVAL (nmat or V < 1, NULL pointers), MD_EUNSUPPORTED (d not
 * a positive multiple of 8), MD_EHIP. */
int md_vocab_tile_norms(int nmat, int V, int d, const void* U, float* norms, void* stream);

/* The draft heads and their top-k lists.
 *
 * Medusa (kind = MD_HEADS_MEDUSA, level = 0): for every row m < M of
 * h [M][d] (device, dt) and every head k < K:
 *     h'_k[m] = h[m] + SiLU(W[k] h[m] + b[k])      W [K][d][d], b [K][d]
 *     logit   = U[k] h'_k[m]                       U [K][V][d]   (device, dt)
 * topk_idx[m][k][j], topk_val[m][k][j] (device int32 / float32, [M][K][kmax])
 * receive the k_per_head[k] best logits ordered by value descending, equal
 * values by index ascending; entries j >= k_per_head[k] are -1 / -inf.
 * h' enters the projection in float32 (with 8 or more bf16 rows, as the sum
 * of two bf16 terms hi + lo, |h' - hi - lo| <= 2^-17 |h'|).
 *
 * Medusa with one shared projection (kind = MD_HEADS_MEDUSA_SHARED, level =
 * 0; "What interviewers probe next": the heads keep their residual blocks
 * and use a single vocabulary matrix): as Medusa, with logit = U h'_k[m] for
 * every head and U [V][d]. The K M vectors h' share one pass over U.
 *
 * Hydra (kind = MD_HEADS_HYDRA, level = i in 1..K): head i-1 only, one row per
 * (request b < M, parent p at depth i-1 that has children in `tree`, in node
 * order): x = [h[b] ; E[tok(p)]] with tok(root) = root_tok[b] and
 * tok(p) = tree_tok[b][p] otherwise; h' = h[b] + SiLU(W[i-1] x + b[i-1]) with
 * W [K][d][2d]; logits = U[i-1] h'. Row r = b * P_i + (index of p among the
 * level's parents). Outputs are [rows][1][kmax]. E [V][d] (device, dt),
 * root_tok [M], tree_tok [M][tree->n] (device int32); tree (host). A
 * parent token outside [0, V) reads as a zero embedding.
 *
 * b may be NULL (zero bias). h_res (device float32, optional) receives h'
 * as [K][M][d] (Medusa) or [rows][d] (Hydra). ws (device) must hold
 * md_heads_workspace_bytes(...). k_per_head (host) has K entries in [1, 16],
 * kmax = their maximum. Requires d % 8 == 0, K <= 8.
 *
 * U_op (optional, NULL for none): the operand-order copy of U (bf16 only;
 * md_operand_order over the K matrices [V][d], or the one shared matrix).
 * With it the matrix-core path runs from 2 bf16 rows (else from 8) and its
 * few-row kernels (up to 128 rows) read U_op instead of U; the results are
 * the same bit for bit. MD_EINVAL if given with dt = MD_F32.
 *
 * U_norms (optional, NULL for none): md_vocab_tile_norms of U (the K
 * matrices, or the one shared matrix; bf16 only). The many-row certified pass
 * then takes each tile's row norm from it instead of computing it; the lists
 * are the same (they come from the exact re-scoring either way). MD_EINVAL
 * if given with dt = MD_F32. A table that does not belong to U, or is too
 * small, voids the certificate (undefined results, no fault).
 *
 * W_op (optional, NULL for none): the operand-order copy of W (bf16 only;
 * md_operand_order over the K matrices [d][din], din = d, or 2d for Hydra).
 * The few-row matrix-core residual kernels (up to 16 rows, and 17 to 77 rows
 * at din = 8,192) then read each weight fragment as one consecutive 1 KB;
 * the products and their order are the same, so are the results, bit for
 * bit. MD_EINVAL if given with dt = MD_F32. */
int md_medusa_heads(int kind, int dt, int M, int d, int V, int K, const int32_t* k_per_head, int level,
                    const md_tree* tree, const void* h, const void* W, const void* b, const void* U, const void* U_op,
                    const float* U_norms, const void* W_op, const void* E, const int32_t* root_tok,
                    const int32_t* tree_tok, int32_t* topk_idx, float* topk_val, float* h_res, void* ws,
                    size_t ws_bytes, void* stream);

/* The candidate tree's tokens and positions ("Trees").
 *
 * Medusa (kind = MD_HEADS_MEDUSA or MD_HEADS_MEDUSA_SHARED, level = 0):
 * tree_tok[b][n] = root_tok[b] for
 * the root, else topk_idx[src_row[b]][depth(n) - 1][rank(n)] with topk_idx
 * [M][K][kmax]; tree_pos[b][n] = lens[b] + depth(n). A src_row entry outside
 * [0, M) yields -1 tokens for that request's non-root nodes.
 * Hydra (kind = MD_HEADS_HYDRA, level = i in 1..K): fills the depth-i nodes
 * from the level's lists [rows][1][kmax] (each node reads its own parent's
 * row, as md_medusa_heads numbers them); level 1 also writes the root token
 * and every position. M and src_row are ignored for Hydra (src_row may be
 * NULL). All arrays are device int32; tree_tok, tree_pos are [B][tree->n]. */
int md_tree_build(const md_tree* tree, int kind, int B, int M, int K, int kmax, int level, const int32_t* topk_idx,
                  const int32_t* src_row, const int32_t* root_tok, const int32_t* lens, int32_t* tree_tok,
                  int32_t* tree_pos, void* stream);

/* Workspace for md_tree_attention at these sizes (max_len bounds lens). */
size_t md_attention_workspace_bytes(int dt, int B, int N, int Hq, int Hkv, int hd, int max_len);

/* Tree-masked attention of every node over the KV cache, in one pass.
 *
 * q [B][N][Hq][hd], out [B][N][Hq][hd] (device, dt); Kc, Vc [B][Hkv][Lcap][hd]
 * (device, dt) hold the cached keys/values in slots [0, lens[b]) and the tree
 * nodes' own keys/values in slots lens[b] + n. Node n, query head h attends
 * to slots [0, lens[b]) and to lens[b] + j for every j that is n or an
 * ancestor of n; it reads kv head h / (Hq / Hkv). Weights are
 * softmax(scale * q.k). lens (device int32 [B]) must lie in [0, max_len]
 * with max_len + N <= Lcap (values above max_len are read as max_len).
 * Requires Hq % Hkv == 0, hd in {64, 128}. No positional encoding is applied:
 * q and k are taken as already encoded. */
int md_tree_attention(const md_tree* tree, int dt, int B, int Hq, int Hkv, int hd, int Lcap, int max_len,
                      const void* q, const void* Kc, const void* Vc, const int32_t* lens, float scale, void* out,
                      void* ws, size_t ws_bytes, void* stream);

/* md_tree_attention for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same inputs, outputs, checks and errors, no workspace
 * argument. The key ranges' partial rows live in one static scratch array
 * per GPU inside the library (md_tree_attention_noalloc_max_bytes() bytes,
 * 32 MiB, held from the library's first use on that GPU until the process
 * ends); the call allocates and frees nothing. Sizes whose workspace
 * (md_attention_workspace_bytes) exceeds it return MD_EWORKSPACE. Every
 * call on one GPU uses the same array: calls that overlap on one GPU (other
 * streams, other threads) race, so serialise them. The first call on a GPU
 * looks up the array's device address there (MD_EHIP if that fails). */
int md_tree_attention_noalloc(const md_tree* tree, int dt, int B, int Hq, int Hkv, int hd, int Lcap, int max_len,
                              const void* q, const void* Kc, const void* Vc, const int32_t* lens, float scale,
                              void* out, void* stream);
size_t md_tree_attention_noalloc_max_bytes(void);

/* Workspace for md_tree_accept. */
size_t md_accept_workspace_bytes(int B, int N, int V);

/* Greedy verification, acceptance and cache compaction.
 *
 * t*(b, n) = the first index of the maximum of logits[b][n][:] (device
 * float32 [B][N][V]). A non-root node c matches when tree_tok[b][c] equals
 * t* at its parent; a node is accepted when it and all its non-root
 * ancestors match. With a the deepest accepted node (lowest index among
 * equals): accept_len[b] = depth(a) + 1, path[b][j] = a's ancestor at depth j
 * (-1 padded to K + 1), next_tok[b] = t*(b, a), compact_src[b][j] =
 * lens[b] + path[b][j] (-1 padded). Then, for j < accept_len[b], cache slot
 * lens[b] + j of K and V takes what slot lens[b] + path[b][j] held before
 * the call (all kv heads), and lens[b] grows by accept_len[b]. Slots below
 * lens[b] are untouched. K is the number of heads (the tree's depth <= K).
 * Outputs are device int32: accept_len, next_tok [B]; path, compact_src
 * [B][K + 1]. Kc, Vc, lens are updated in place. */
int md_tree_accept(const md_tree* tree, int dt, int B, int K, int V, int Hkv, int hd, int Lcap,
                   const float* logits, const int32_t* tree_tok, void* Kc, void* Vc, int32_t* lens,
                   int32_t* accept_len, int32_t* path, int32_t* next_tok, int32_t* compact_src, void* ws,
                   size_t ws_bytes, void* stream);

/* Workspace for md_target_argmax at these sizes. */
size_t md_target_argmax_workspace_bytes(int dt, int R, int d, int V);

/* The target's greedy choice at every tree node from its final hidden
 * states: the last step of the one verification pass ("Trees"), the target's
 * LM head, with the argmax fused so the R x V logits never reach memory.
 *     tok[r] = the first index of the maximum over v of Wt[v] . H[r]
 *     val[r] = that maximum
 * H [R][d] (device, dt; for a step R = B * N rows in (request, node) order),
 * Wt [V][d] (device, dt), tok [R] (device int32), val [R] (device float32,
 * or NULL). Products of the stored values are exact and summed in float32.
 * ws (device) must hold md_target_argmax_workspace_bytes(...). Wt_op
 * (optional, NULL for none): the operand-order copy of Wt (bf16 only, see
 * md_operand_order); with it 2 to 128 rows run on the matrix cores reading
 * Wt_op, with the same results. Requires d % 8 == 0 and d * 4 bytes <=
 * 160 KB. Errors: MD_EINVAL (negative sizes, NULL pointers, unknown dt,
 * Wt_op with MD_F32), MD_EUNSUPPORTED (d), MD_EWORKSPACE. */
int md_target_argmax(int dt, int R, int d, int V, const void* H, const void* Wt, const void* Wt_op, int32_t* tok,
                     float* val, void* ws, size_t ws_bytes, void* stream);

/* md_tree_accept with the target's choices given instead of its logits:
 * target_tok [B][N] (device int32; t*(b, n), e.g. from md_target_argmax).
 * Same outputs, cache update and errors; no workspace. */
int md_tree_accept_tokens(const md_tree* tree, int dt, int B, int K, int Hkv, int hd, int Lcap,
                          const int32_t* target_tok, const int32_t* tree_tok, void* Kc, void* Vc, int32_t* lens,
                          int32_t* accept_len, int32_t* path, int32_t* next_tok, int32_t* compact_src, void* stream);

/* ---------------------------------------------------------------- sampled decoding
 *
 * "Medusa heads versus separate draft model", section "Training": with
 * sampling at a temperature T, rejection sampling with the heads'
 * probabilities keeps the target's distribution exactly; "typical
 * acceptance" takes more drafts and does not. The pages give neither rule on
 * a tree; the calls below implement these readings:
 *   q_i = softmax(l_i / T) is head i's draft distribution, p_n =
 *   softmax(target_logits[n] / T) the target's at node n;
 *   head i's draft tokens are k_i distinct tokens drawn from q_i without
 *   replacement, in draw order (md_draft_sample); they fill the tree exactly
 *   as top-k lists do (md_tree_build);
 *   verification (md_tree_verify_sampled) walks from the root and tries a
 *   node's children in rank order, accepting child x with probability
 *   min(1, p(x) / q(x)); on rejection p <- normalise(max(0, p - q)) and x
 *   leaves q (renormalised). An accepted child becomes the node; with every
 *   child rejected, or at a leaf, the step's last token is drawn from p;
 *   typical acceptance (md_tree_accept_typical): node n matches when its
 *   parent's p gives tok(n) more than min(eps, delta * exp(-H(p))), H the
 *   entropy; the deepest node whose root path matches (lowest index among
 *   equals) ends the step and its p gives the last token;
 *   a tree token outside [0, V) is never accepted and changes nothing.
 * Random numbers are inputs: 32-bit words w give uniforms
 * u = (floor(w / 2^9) + 1/2) * 2^-23 in (0, 1) and Gumbel noise -log(-log u);
 * draws from a distribution are Gumbel-max (the largest log-probability plus
 * noise), ties to the lowest index. The caller supplies fresh words for every
 * step. Temperatures must be positive and finite. */

/* Workspace for md_medusa_heads_logits. */
size_t md_heads_logits_workspace_bytes(int kind, int M, int d, int K);

/* md_medusa_heads (Medusa kinds only) writing every logit instead of the top-k:
 * logits [M][K][V] (device float32), logits[m][i][v] = U_i[v] . h'_i(m).
 * Same inputs, checks and errors; the GEMV path at any M. */
int md_medusa_heads_logits(int kind, int dt, int M, int d, int V, int K, const void* h, const void* W, const void* b,
                           const void* U, float* logits, float* h_res, void* ws, size_t ws_bytes, void* stream);

/* Workspace for md_draft_sample. */
size_t md_draft_sample_workspace_bytes(int M, int K, int V, int kmax);

/* Draft tokens drawn from the heads: for every (row m, head i), the k_i
 * largest of logits[m][i][v] / T + G(words[m][i][v]) by (value desc, index
 * asc), i.e. k_i distinct tokens drawn without replacement from
 * softmax(logits / T) in draw order, written to tok[m][i][0..k_i) (device
 * int32 [M][K][kmax], -1 padded; the layout of md_medusa_heads' topk_idx),
 * and lse[m][i] = log sum_v exp(logits[m][i][v] / T) (device float32 [M][K]).
 * logits, words: device [M][K][V]. Errors: MD_EINVAL (sizes, k_per_head
 * outside 1..16 or above V, T not positive, NULL pointers), MD_EWORKSPACE. */
int md_draft_sample(int M, int K, int V, const int32_t* k_per_head, float temperature, const float* logits,
                    const uint32_t* words, int32_t* tok, float* lse, void* ws, size_t ws_bytes, void* stream);

/* Workspace for md_tree_verify_sampled. */
size_t md_verify_sampled_workspace_bytes(int B, int N);

/* Rejection-sampling verification, acceptance and cache compaction.
 * target_logits [B][N][V] (device float32: the target at every node);
 * head_logits [B][K][V] and head_lse [B][K] (device float32: the heads that
 * drafted request b's tree and their log-sum-exp at T, as md_draft_sample
 * gives them); u_words [B][N] (device uint32: word of node n's acceptance
 * test); g_words [B][V] (device uint32: the last token's draw). The accepted
 * path, accept_len, path, next_tok (the step's last token), compact_src and
 * the cache update are as md_tree_accept defines them for the path this walk
 * takes. Errors as md_tree_accept's, and MD_EINVAL for T. */
int md_tree_verify_sampled(const md_tree* tree, int dt, int B, int K, int V, int Hkv, int hd, int Lcap,
                           float temperature, const float* target_logits, const float* head_logits,
                           const float* head_lse, const int32_t* tree_tok, const uint32_t* u_words,
                           const uint32_t* g_words, void* Kc, void* Vc, int32_t* lens, int32_t* accept_len,
                           int32_t* path, int32_t* next_tok, int32_t* compact_src, void* ws, size_t ws_bytes,
                           void* stream);

/* Workspace for md_tree_accept_typical. */
size_t md_accept_typical_workspace_bytes(int B, int N);

/* Typical acceptance, acceptance and cache compaction (not exact in
 * distribution). target_logits [B][N][V] (device float32), g_words [B][V]
 * (device uint32: the last token's draw at the final node); eps, delta >= 0.
 * Outputs and cache update as md_tree_accept defines them for the node this
 * rule picks. Errors as md_tree_accept's, and MD_EINVAL for T, eps, delta. */
int md_tree_accept_typical(const md_tree* tree, int dt, int B, int K, int V, int Hkv, int hd, int Lcap,
                           float temperature, float eps, float delta, const float* target_logits,
                           const int32_t* tree_tok, const uint32_t* g_words, void* Kc, void* Vc, int32_t* lens,
                           int32_t* accept_len, int32_t* path, int32_t* next_tok, int32_t* compact_src, void* ws,
                           size_t ws_bytes, void* stream);

/* Testing hook for the single-launch heads kernel (md_heads_fused): the
 * number of polls each of its two bounded waits makes on this thread's later
 * md_medusa_heads calls before giving up (-1: the built-in limits, tens to
 * hundreds of milliseconds). With residual_polls = 0 every block computes
 * its head's h' alone instead of waiting for its group's (slow; the same
 * results); with list_polls = 0 each head's merging block gives up at once
 * and writes -1 indices and -inf values for its head (a failure the caller
 * can see). Errors: MD_EINVAL for values below -1. */
int md_set_wait_limits(int residual_polls, int list_polls);

/* Timing hook for profiling: when both are non-NULL hipEvent_t handles, every
 * later md_medusa_heads or md_medusa_heads_logits call on this thread records
 * `start` on its stream right before its vocabulary-projection kernel and
 * `stop` right after it.
 * Pass NULL, NULL to stop. */
int md_set_vocab_timing_events(void* start, void* stop);

/* Measurement utility, not a step of the method: streams `bytes` bytes of
 * device memory `buf` once with 16-byte non-temporal loads spread over the
 * whole GPU, and writes one word per block to `sink` (device, uint32,
 * md_hbm_read_probe_blocks() entries). It gives the attainable HBM read
 * bandwidth of the running GPU and a kernel of known traffic for scaling
 * hardware byte counters. bytes must be a positive multiple of 16 and buf
 * 16-byte aligned. */
int md_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream);
int md_hbm_read_probe_blocks(void);

/* Thread-local text for the last non-MD_OK return on this thread. */
const char* md_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MEDUSA_H */
