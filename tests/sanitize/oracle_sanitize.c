/*
 * Drives every exported function of the CPU oracle (oracle/oracle.c) and of
 * the input generator (synth/synth.c) once on small inputs held in buffers of
 * exactly the size each call may touch, so that a build with
 * -fsanitize=address,undefined reports any read or write past a buffer, any
 * use after free and any undefined arithmetic. It also checks a few results
 * that hold by definition, and exits non-zero on the first failure.
 * Test infrastructure only (built and run by tests/test_sanitize_cpu.py).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void syn_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]);
void syn_normal_f32(uint64_t seed, uint32_t stream, int64_t first, int64_t n, double std_, float* out);
void syn_normal_bf16(uint64_t seed, uint32_t stream, int64_t first, int64_t n, double std_, uint16_t* out);
void syn_u32(uint64_t seed, uint32_t stream, int64_t first, int64_t n, uint32_t* out);

void orc_set_threads(int t);
int orc_get_threads(void);
void orc_to_double(int dt, int64_t n, const void* src, double* dst);
int64_t orc_head_weight_elems(int din, int d, int V);
void orc_residual(int dt, int M, int din, int d, const double* x, const double* base, const void* W,
                  const void* b, double* hres);
void orc_vocab_topk(int dt, int M, int d, int V, const double* hres, const void* U, int k, int32_t* idx,
                    double* val, double* margin, double* logits_out);
void orc_tree_tokens_medusa(int N, const int8_t* parent, const int8_t* rank, int B, int K, int kmax,
                            const int32_t* topk_idx, const int32_t* src_row, const int32_t* root_tok,
                            const int32_t* lens, int32_t* tree_tok, int32_t* tree_pos);
void orc_tree_attention(int dt, int B, int N, const int8_t* parent, int Hq, int Hkv, int hd, int Lcap,
                        const void* q, const void* Kc, const void* Vc, const int32_t* lens, double scale,
                        double* out);
void orc_argmax(int64_t R, int V, const float* logits, int32_t* out);
void orc_accept(int N, const int8_t* parent, int B, int K, const int32_t* tree_tok, const int32_t* tstar,
                const int32_t* lens, int32_t* accept_len, int32_t* path, int32_t* next_tok,
                int32_t* compact_src);
void orc_compact(int dt, int B, int Hkv, int hd, int Lcap, void* Kc, void* Vc, int32_t* lens,
                 const int32_t* accept_len, const int32_t* path, int K);

#define CHECK(c)                                                      \
    do {                                                              \
        if (!(c)) {                                                   \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            exit(1);                                                  \
        }                                                             \
    } while (0)

static void* xmalloc(size_t n) {
    void* p = malloc(n ? n : 1);
    CHECK(p != NULL);
    return p;
}

/* the 7-node tree: root; depth 1 ranks 0, 1; under rank 0 ranks 0, 1; under
 * rank 1 rank 0; a depth-3 node under (0, 0) */
static const int8_t PARENT[7] = {-1, 0, 0, 1, 1, 2, 3};
static const int8_t RANK[7] = {0, 0, 1, 0, 1, 0, 0};
enum { N = 7, K = 3, KMAX = 2 };

int main(void) {
    orc_set_threads(1);
    CHECK(orc_get_threads() == 1);

    /* generator: every entry point, odd first/n so the block edges are hit */
    uint32_t ctr[4] = {0, 0, 0, 0}, key[2] = {0, 0}, w4[4];
    syn_philox4x32_10(ctr, key, w4);
    float* f = (float*)xmalloc(7 * sizeof(float));
    syn_normal_f32(1, 2, 3, 7, 1.0, f);
    uint16_t* hb = (uint16_t*)xmalloc(5 * sizeof(uint16_t));
    syn_normal_bf16(1, 3, 1, 5, 0.5, hb);
    uint32_t* u = (uint32_t*)xmalloc(9 * sizeof(uint32_t));
    syn_u32(4, 5, 2, 9, u);
    syn_u32(4, 5, 0, 0, u); /* empty range writes nothing */
    double* fd = (double*)xmalloc(7 * sizeof(double));
    orc_to_double(0, 7, f, fd);
    for (int i = 0; i < 7; ++i) CHECK(fd[i] == (double)f[i]);
    double* hd5 = (double*)xmalloc(5 * sizeof(double));
    orc_to_double(1, 5, hb, hd5);
    CHECK(orc_head_weight_elems(16, 16, 40) == 16 * 16 + 16 + 16 * 40);

    /* heads: a Hydra-shaped residual (din = 2d) in bf16 and f32, then the
     * projection with k = V (the margin loop's last element) and k = 1 */
    const int M = 2, d = 16, din = 2 * d, V = 40;
    uint16_t* Wb = (uint16_t*)xmalloc((size_t)d * din * 2);
    syn_normal_bf16(7, 1, 0, (int64_t)d * din, 0.2, Wb);
    uint16_t* bb = (uint16_t*)xmalloc((size_t)d * 2);
    syn_normal_bf16(7, 2, 0, d, 0.2, bb);
    float* Wf = (float*)xmalloc((size_t)d * din * 4);
    syn_normal_f32(7, 1, 0, (int64_t)d * din, 0.2, Wf);
    double* x = (double*)xmalloc((size_t)M * din * 8);
    double* base = (double*)xmalloc((size_t)M * d * 8);
    for (int i = 0; i < M * din; ++i) x[i] = sin(0.37 * i);
    for (int i = 0; i < M * d; ++i) base[i] = cos(0.11 * i);
    double* hres = (double*)xmalloc((size_t)M * d * 8);
    orc_residual(1, M, din, d, x, base, Wb, bb, hres);
    orc_residual(0, M, din, d, x, base, Wf, NULL, hres);
    uint16_t* Ub = (uint16_t*)xmalloc((size_t)V * d * 2);
    syn_normal_bf16(7, 3, 0, (int64_t)V * d, 0.25, Ub);
    int32_t* idx = (int32_t*)xmalloc((size_t)M * V * 4);
    double* val = (double*)xmalloc((size_t)M * V * 8);
    double* margin = (double*)xmalloc((size_t)M * 8);
    double* logits = (double*)xmalloc((size_t)M * V * 8);
    orc_vocab_topk(1, M, d, V, hres, Ub, V, idx, val, margin, logits);
    for (int m = 0; m < M; ++m)
        for (int j = 0; j + 1 < V; ++j) CHECK(val[m * V + j] >= val[m * V + j + 1]);
    orc_vocab_topk(1, M, d, V, hres, Ub, 1, idx, val, margin, NULL);

    /* tree tokens from [M][K][KMAX] lists, two requests */
    const int B = 2;
    int32_t* lists = (int32_t*)xmalloc((size_t)M * K * KMAX * 4);
    for (int i = 0; i < M * K * KMAX; ++i) lists[i] = (i * 7) % V;
    int32_t src_row[2] = {1, 0}, root_tok[2] = {3, 9}, lens[2] = {0, 5};
    int32_t* tok = (int32_t*)xmalloc((size_t)B * N * 4);
    int32_t* pos = (int32_t*)xmalloc((size_t)B * N * 4);
    orc_tree_tokens_medusa(N, PARENT, RANK, B, K, KMAX, lists, src_row, root_tok, lens, tok, pos);
    CHECK(tok[0] == 3 && tok[N] == 9 && pos[N + 6] == 5 + 3);

    /* attention: Lcap exactly max(lens) + N, an empty cache for request 0 */
    const int Hq = 4, Hkv = 2, hdim = 8, Lcap = 5 + N;
    size_t nq = (size_t)B * N * Hq * hdim, nkv = (size_t)B * Hkv * Lcap * hdim;
    uint16_t* q = (uint16_t*)xmalloc(nq * 2);
    uint16_t* Kc = (uint16_t*)xmalloc(nkv * 2);
    uint16_t* Vc = (uint16_t*)xmalloc(nkv * 2);
    syn_normal_bf16(8, 1, 0, (int64_t)nq, 1.0, q);
    syn_normal_bf16(8, 2, 0, (int64_t)nkv, 1.0, Kc);
    syn_normal_bf16(8, 3, 0, (int64_t)nkv, 1.0, Vc);
    double* out = (double*)xmalloc(nq * 8);
    orc_tree_attention(1, B, N, PARENT, Hq, Hkv, hdim, Lcap, q, Kc, Vc, lens, 1.0 / sqrt(hdim), out);
    /* request 0's root sees one key (its own slot 0): out = that v */
    for (int h = 0; h < Hq; ++h)
        for (int c = 0; c < hdim; ++c) {
            int g = h / (Hq / Hkv);
            uint32_t bits = (uint32_t)Vc[((size_t)g * Lcap + 0) * hdim + c] << 16;
            float v;
            memcpy(&v, &bits, 4);
            CHECK(fabs(out[(size_t)h * hdim + c] - v) < 1e-12);
        }

    /* verification: request 0 accepts the (0, 0, 0) chain, request 1 nothing */
    const int Vt = 40;
    float* tl = (float*)xmalloc((size_t)B * N * Vt * 4);
    syn_normal_f32(9, 1, 0, (int64_t)B * N * Vt, 1.0, tl);
    for (int n = 0; n < N; ++n) {
        int child = n == 0 ? 1 : n == 1 ? 3 : n == 3 ? 6 : -1;
        if (child >= 0) tl[(size_t)n * Vt + tok[child]] = 100.0f;
    }
    int32_t* ts = (int32_t*)xmalloc((size_t)B * N * 4);
    /* request 1: every row's maximum is token Vt - 1, which no list holds */
    for (int n = 0; n < N; ++n) tl[(size_t)(N + n) * Vt + Vt - 1] = 100.0f;
    orc_argmax((int64_t)B * N, Vt, tl, ts);
    for (int n = 0; n < N; ++n) CHECK(ts[N + n] == Vt - 1);
    for (int c = 1; c < N; ++c) CHECK(tok[N + c] != Vt - 1);
    int32_t acc[2], path[2 * (K + 1)], nxt[2], csrc[2 * (K + 1)];
    orc_accept(N, PARENT, B, K, tok, ts, lens, acc, path, nxt, csrc);
    CHECK(acc[0] == K + 1 && path[0] == 0 && path[1] == 1 && path[2] == 3 && path[3] == 6);
    CHECK(acc[1] == 1 && path[K + 1] == 0 && path[K + 2] == -1 && csrc[K + 1] == 5);

    /* compaction: sources are later destinations (slot 3 -> 2, 6 -> 3) */
    uint16_t* K0 = (uint16_t*)xmalloc(nkv * 2);
    memcpy(K0, Kc, nkv * 2);
    int32_t lens2[2] = {lens[0], lens[1]};
    orc_compact(1, B, Hkv, hdim, Lcap, Kc, Vc, lens2, acc, path, K);
    CHECK(lens2[0] == K + 1 && lens2[1] == 5 + 1);
    for (int g = 0; g < Hkv; ++g)
        for (int j = 0; j < K + 1; ++j)
            CHECK(memcmp(Kc + ((size_t)g * Lcap + j) * hdim, K0 + ((size_t)g * Lcap + path[j]) * hdim, hdim * 2) == 0);

    free(f); free(hb); free(u); free(fd); free(hd5); free(Wb); free(bb); free(Wf); free(x); free(base);
    free(hres); free(Ub); free(idx); free(val); free(margin); free(logits); free(lists); free(tok);
    free(pos); free(q); free(Kc); free(Vc); free(out); free(tl); free(ts); free(K0);
    printf("sanitized oracle and generator: all calls clean\n");
    return 0;
}
