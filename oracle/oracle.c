/*
 * CPU oracle for the Medusa tree-decode step. TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the bench's CPU-baseline leg load this
 * library. The GPU library never links, calls or reads it, and it shares no
 * source with the GPU library.
 *
 * Every function is the plain definition written out in double precision:
 * loops in the order the definition states them, one output per loop
 * iteration, no blocking, no fusion. Inputs arrive in their storage type
 * (dt = 0: float32, dt = 1: bfloat16 bit patterns) and are converted to
 * double exactly. OpenMP only splits independent outputs across threads,
 * so results do not depend on the thread count. Build with gcc -O2
 * -ffp-contract=off (no fast-math, no fused multiply-add).
 *
 * Sources (the pages):
 *  [P1] "Medusa heads versus separate draft model" (inferenceinterviews.com):
 *       "What each one is" (heads on the last hidden state, a residual block
 *       then a vocabulary projection per head), "Cost per step" (parameter
 *       counts), "Acceptance" (table and the closed form of E), "Trees"
 *       (top few per head, tree of combinations, one pass with a tree
 *       attention mask, advance along the branch that matches).
 *  [P3/P4] Hydra summary and abstract (study.space; codewithpapers.app):
 *       sequentially dependent heads that also see the preceding speculated
 *       token.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- helpers */

static double bf16_bits_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static double elem(const void* p, int dt, int64_t i) {
    return dt == 0 ? (double)((const float*)p)[i] : bf16_bits_to_double(((const uint16_t*)p)[i]);
}

/* SiLU(x) = x * sigmoid(x) = x / (1 + e^-x). */
static double silu(double x) { return x / (1.0 + exp(-x)); }

static int node_depth(const int8_t* parent, int n) {
    int d = 0;
    while (parent[n] >= 0) {
        n = parent[n];
        ++d;
    }
    return d;
}

/* Is node j node n itself or one of n's ancestors? (walks the parent links) */
static int is_anc_or_self(const int8_t* parent, int j, int n) {
    for (int c = n; c >= 0; c = parent[c])
        if (c == j) return 1;
    return 0;
}

void orc_set_threads(int t) {
#ifdef _OPENMP
    if (t > 0) omp_set_num_threads(t);
#else
    (void)t;
#endif
}

int orc_get_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void orc_to_double(int dt, int64_t n, const void* src, double* dst) {
    for (int64_t i = 0; i < n; ++i) dst[i] = elem(src, dt, i);
}

/* Number of weight elements one head's loops read: [P1] "Cost per step"
 * counts a d x d residual matrix plus a bias plus a d x V projection. With
 * Hydra's concatenated input the residual matrix is d x 2d. */
int64_t orc_head_weight_elems(int din, int d, int V) {
    int64_t n = 0;
    n += (int64_t)d * din; /* W, one element per (r, c) of orc_residual */
    n += d;                /* bias b */
    n += (int64_t)V * d;   /* U, one element per (v, c) of orc_vocab_topk */
    return n;
}

/* ------------------------------------------------------- residual block */

/* [P1] "What each one is": a head is one residual block on the hidden state.
 * For every row m and output r:
 *     z        = sum_c W[r][c] * x[m][c] + b[r]
 *     hres[m][r] = base[m][r] + SiLU(z)
 * Medusa: x = base = h (din = d). Hydra [P3/P4]: x = [h ; E[parent token]]
 * (din = 2d) and base = h. b may be NULL (zero bias). */
void orc_residual(int dt, int M, int din, int d, const double* x, const double* base,
                  const void* W, const void* b, double* hres) {
    for (int m = 0; m < M; ++m) {
#pragma omp parallel for schedule(static)
        for (int r = 0; r < d; ++r) {
            double z = 0.0;
            for (int c = 0; c < din; ++c) z += elem(W, dt, (int64_t)r * din + c) * x[(int64_t)m * din + c];
            z += b ? elem(b, dt, r) : 0.0;
            hres[(int64_t)m * d + r] = base[(int64_t)m * d + r] + silu(z);
        }
    }
}

/* ------------------------------------------ vocabulary projection + top-k */

typedef struct {
    double v;
    int32_t i;
} scored;

/* total order: larger value first; equal values -> lower index first */
static int cmp_scored(const void* a, const void* b) {
    const scored* x = (const scored*)a;
    const scored* y = (const scored*)b;
    if (x->v > y->v) return -1;
    if (x->v < y->v) return 1;
    return (x->i > y->i) - (x->i < y->i);
}

/* [P1] "What each one is" (each head has its own d x V projection) and
 * "Trees" (take the top few candidates of each head):
 *     logit[v] = sum_c U[v][c] * hres[m][c]
 * then every logit is sorted by (value desc, index asc) and the first k kept.
 * margin[m] = the smallest gap between consecutive sorted values among the
 * first k + 1, i.e. how far the list is from changing order or membership.
 * logits_out (optional, [M][V]) receives the unsorted logits. */
void orc_vocab_topk(int dt, int M, int d, int V, const double* hres, const void* U, int k,
                    int32_t* idx, double* val, double* margin, double* logits_out) {
    scored* s = (scored*)malloc(sizeof(scored) * (size_t)V);
    for (int m = 0; m < M; ++m) {
        const double* x = hres + (int64_t)m * d;
#pragma omp parallel for schedule(static)
        for (int v = 0; v < V; ++v) {
            double acc = 0.0;
            for (int c = 0; c < d; ++c) acc += elem(U, dt, (int64_t)v * d + c) * x[c];
            s[v].v = acc;
            s[v].i = v;
            if (logits_out) logits_out[(int64_t)m * V + v] = acc;
        }
        qsort(s, (size_t)V, sizeof(scored), cmp_scored);
        double mg = INFINITY;
        for (int j = 0; j < k; ++j) {
            idx[(int64_t)m * k + j] = s[j].i;
            val[(int64_t)m * k + j] = s[j].v;
            if (j + 1 < V) {
                double gap = s[j].v - s[j + 1].v;
                if (gap < mg) mg = gap;
            }
        }
        margin[m] = mg;
    }
    free(s);
}

/* ------------------------------------------------------------ tree build */

/* [P1] "Trees": the tree holds combinations of the heads' candidates. Node n
 * at depth j >= 1 carries entry rank[n] of head j's list for the row that
 * builds request b's tree; the root carries the target's own next token.
 * Position = cached length + depth.
 * topk_idx is [M][K][kmax]. */
void orc_tree_tokens_medusa(int N, const int8_t* parent, const int8_t* rank, int B, int K, int kmax,
                            const int32_t* topk_idx, const int32_t* src_row, const int32_t* root_tok,
                            const int32_t* lens, int32_t* tree_tok, int32_t* tree_pos) {
    for (int b = 0; b < B; ++b) {
        for (int n = 0; n < N; ++n) {
            int dep = node_depth(parent, n);
            int32_t tok;
            if (n == 0)
                tok = root_tok[b];
            else
                tok = topk_idx[((int64_t)src_row[b] * K + (dep - 1)) * kmax + rank[n]];
            tree_tok[b * N + n] = tok;
            tree_pos[b * N + n] = lens[b] + dep;
        }
    }
}

/* ------------------------------------------------------- tree attention */

/* [P1] "Trees": every node is verified in one pass under a tree attention
 * mask. Node n, query head h of request b attends to the cached keys
 * [0, L_b) and to the tree's own keys in slots L_b + j for every node j that
 * is n or an ancestor of n. Query head h reads kv head h / (Hq / Hkv).
 *     s_i = scale * q . k_i;  out = sum_i e^{s_i - max} v_i / sum_i e^{s_i - max}
 * q, out: [B][N][Hq][hd]; Kc, Vc: [B][Hkv][Lcap][hd]. */
void orc_tree_attention(int dt, int B, int N, const int8_t* parent, int Hq, int Hkv, int hd, int Lcap,
                        const void* q, const void* Kc, const void* Vc, const int32_t* lens, double scale,
                        double* out) {
    int group = Hq / Hkv;
    int64_t total = (int64_t)B * N * Hq;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < total; ++t) {
        int b = (int)(t / ((int64_t)N * Hq));
        int n = (int)((t / Hq) % N);
        int h = (int)(t % Hq);
        int g = h / group;
        int L = lens[b];
        int nk = 0;
        int* slot = (int*)malloc(sizeof(int) * (size_t)(L + N));
        for (int i = 0; i < L; ++i) slot[nk++] = i;
        for (int j = 0; j < N; ++j)
            if (is_anc_or_self(parent, j, n)) slot[nk++] = L + j;
        double* s = (double*)malloc(sizeof(double) * (size_t)nk);
        int64_t qoff = (((int64_t)b * N + n) * Hq + h) * hd;
        int64_t kvoff = ((int64_t)b * Hkv + g) * Lcap;
        double mx = -INFINITY;
        for (int i = 0; i < nk; ++i) {
            double acc = 0.0;
            for (int c = 0; c < hd; ++c) acc += elem(q, dt, qoff + c) * elem(Kc, dt, (kvoff + slot[i]) * hd + c);
            s[i] = scale * acc;
            if (s[i] > mx) mx = s[i];
        }
        double Z = 0.0;
        for (int i = 0; i < nk; ++i) {
            s[i] = exp(s[i] - mx);
            Z += s[i];
        }
        for (int c = 0; c < hd; ++c) {
            double acc = 0.0;
            for (int i = 0; i < nk; ++i) acc += s[i] * elem(Vc, dt, (kvoff + slot[i]) * hd + c);
            out[qoff + c] = acc / Z;
        }
        free(s);
        free(slot);
    }
}

/* ------------------------------------------------ verification and accept */

/* The target's greedy choice per row: the first index of the row maximum. */
void orc_argmax(int64_t R, int V, const float* logits, int32_t* out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        const float* x = logits + r * V;
        int best = 0;
        for (int v = 1; v < V; ++v)
            if (x[v] > x[best]) best = v;
        out[r] = best;
    }
}

/* [P1] "Trees" (if a branch matches, the step advances along it) and
 * "Acceptance" (E counts the target's own token plus the accepted drafts).
 * A non-root node c matches when its token equals the target's choice at its
 * parent; a node is accepted when it and all its non-root ancestors match.
 * The accepted node of greatest depth (lowest index among equals) ends the
 * step: accept_len = its depth + 1, path = its root path in depth order
 * (-1 padded to K + 1), next_tok = the target's choice at it, and
 * compact_src[j] = L_b + path[j] names the cache slot that moves to L_b + j. */
void orc_accept(int N, const int8_t* parent, int B, int K, const int32_t* tree_tok, const int32_t* tstar,
                const int32_t* lens, int32_t* accept_len, int32_t* path, int32_t* next_tok,
                int32_t* compact_src) {
    for (int b = 0; b < B; ++b) {
        const int32_t* tok = tree_tok + (int64_t)b * N;
        const int32_t* ts = tstar + (int64_t)b * N;
        int best = 0, bestd = 0;
        for (int n = 0; n < N; ++n) {
            int ok = 1;
            for (int c = n; c > 0; c = parent[c])
                if (tok[c] != ts[parent[c]]) ok = 0;
            int dep = node_depth(parent, n);
            if (ok && dep > bestd) {
                best = n;
                bestd = dep;
            }
        }
        accept_len[b] = bestd + 1;
        for (int j = 0; j <= K; ++j) {
            path[(int64_t)b * (K + 1) + j] = -1;
            compact_src[(int64_t)b * (K + 1) + j] = -1;
        }
        for (int c = best, j = bestd; c >= 0; c = parent[c], --j) path[(int64_t)b * (K + 1) + j] = c;
        for (int j = 0; j <= bestd; ++j)
            compact_src[(int64_t)b * (K + 1) + j] = lens[b] + path[(int64_t)b * (K + 1) + j];
        next_tok[b] = ts[best];
    }
}

/* Advancing along the accepted branch leaves its cache entries in path
 * order right after the prefix: slot L_b + j takes slot L_b + path[j] for
 * j < accept_len, for K and V of every kv head. All sources are copied out
 * before anything is written. lens[b] grows by accept_len[b]. */
void orc_compact(int dt, int B, int Hkv, int hd, int Lcap, void* Kc, void* Vc, int32_t* lens,
                 const int32_t* accept_len, const int32_t* path, int K) {
    size_t esz = dt == 0 ? 4 : 2;
    for (int b = 0; b < B; ++b) {
        int A = accept_len[b];
        int L = lens[b];
        for (int g = 0; g < Hkv; ++g) {
            for (int which = 0; which < 2; ++which) {
                char* base = (char*)(which == 0 ? Kc : Vc) + (((int64_t)b * Hkv + g) * Lcap) * hd * esz;
                char* tmp = (char*)malloc((size_t)A * hd * esz);
                for (int j = 0; j < A; ++j)
                    memcpy(tmp + (size_t)j * hd * esz,
                           base + (int64_t)(L + path[(int64_t)b * (K + 1) + j]) * hd * esz, hd * esz);
                for (int j = 0; j < A; ++j)
                    memcpy(base + (int64_t)(L + j) * hd * esz, tmp + (size_t)j * hd * esz, hd * esz);
                free(tmp);
            }
        }
        lens[b] = L + A;
    }
}
