// libmedusa C-ABI: argument checks, tree expansion and kernel dispatch.
//
// Every check below runs on the host before any HIP call, so a rejected call
// enqueues nothing. The library holds no device memory besides one static
// scratch array per GPU (md_tree_attention_noalloc), and no state besides
// that array's per-device address, a thread-local error string and the
// optional thread-local timing events.
#include <hip/hip_runtime.h>

#include <atomic>
#include <chrono>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <random>
#include <string>

#include "../../include/medusa.h"
#include "md_internal.h"

namespace {

thread_local std::string g_err;
thread_local hipEvent_t g_ev0 = nullptr, g_ev1 = nullptr;
thread_local int g_spin_res = -1, g_spin_lists = -1;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int hip_status(hipError_t e, const char* where) {
    if (e == hipSuccess) return MD_OK;
    return fail(MD_EHIP, "%s: %s", where, hipGetErrorString(e));
}

// Checks the topology and expands it: depths, ancestor sets, and for Hydra
// the parents of every level. k_per_head may be NULL (ranks unchecked).
int expand_tree(const md_tree* t, int K, const int32_t* k_per_head, DevTree* out) {
    if (!t) return fail(MD_EINVAL, "tree is NULL");
    if (t->n < 1 || t->n > MD_MAX_NODES) return fail(MD_EINVAL, "tree has %d nodes (1..64 supported)", t->n);
    if (K < 1 || K > MD_MAX_HEADS) return fail(MD_EINVAL, "K = %d heads (1..8 supported)", K);
    if (t->parent[0] != -1 || t->rank[0] != 0) return fail(MD_EINVAL, "node 0 must be the root (parent -1, rank 0)");
    DevTree d;
    memset(&d, 0, sizeof(d));
    d.n = t->n;
    d.parent[0] = -1;
    d.depth[0] = 0;
    d.rank[0] = 0;
    d.anc[0] = 1ull;
    int maxd = 0;
    for (int n = 1; n < t->n; ++n) {
        const int p = t->parent[n];
        if (p < 0 || p >= n) return fail(MD_EINVAL, "node %d: parent %d must precede it", n, p);
        const int dep = d.depth[p] + 1;
        if (dep < d.depth[n - 1]) return fail(MD_EINVAL, "node %d: nodes must be numbered breadth-first", n);
        if (dep > K) return fail(MD_EINVAL, "node %d: depth %d exceeds the %d heads", n, dep, K);
        const int r = t->rank[n];
        if (r < 0 || r >= MD_MAX_TOPK) return fail(MD_EINVAL, "node %d: rank %d outside [0, 16)", n, r);
        if (k_per_head && r >= k_per_head[dep - 1])
            return fail(MD_EINVAL, "node %d: rank %d but head %d keeps only %d", n, r, dep, k_per_head[dep - 1]);
        for (int s = 1; s < n; ++s)
            if (t->parent[s] == p && t->rank[s] == r) return fail(MD_EINVAL, "nodes %d and %d: siblings share rank %d", s, n, r);
        d.parent[n] = (int8_t)p;
        d.depth[n] = (int8_t)dep;
        d.rank[n] = (int8_t)r;
        d.anc[n] = d.anc[p] | (1ull << n);
        if (dep > maxd) maxd = dep;
    }
    d.max_depth = maxd;
    // parents per level, in node order
    int off = 0;
    for (int i = 0; i < 64; ++i) d.prow[i] = -1;
    for (int lvl = 1; lvl <= 9; ++lvl) {
        d.level_off[lvl] = off;
        if (lvl <= maxd) {
            int cnt = 0;
            for (int p = 0; p < t->n; ++p) {
                if (d.depth[p] != lvl - 1) continue;
                bool has_child = false;
                for (int c = p + 1; c < t->n; ++c)
                    if (d.parent[c] == p) has_child = true;
                if (!has_child) continue;
                d.lp[off] = (int8_t)p;
                d.prow[p] = (int8_t)cnt;
                ++off;
                ++cnt;
            }
        }
    }
    d.level_off[0] = 0;
    if (out) *out = d;
    return MD_OK;
}

int check_dt(int dt) { return (dt == MD_F32 || dt == MD_BF16) ? MD_OK : fail(MD_EINVAL, "dt = %d (MD_F32 or MD_BF16)", dt); }

}  // namespace

uint64_t launch_token() {
    static std::atomic<uint64_t> next{0};
    static std::once_flag once;
    std::call_once(once, [] {
        std::random_device rd;
        const uint64_t seed = ((uint64_t)rd() << 32) ^ (uint64_t)rd() ^
                              (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
        next.store(seed | 1ull);
    });
    uint64_t t;
    do t = next.fetch_add(1); while (t == 0);
    return t;
}

extern "C" {

const char* md_last_error(void) { return g_err.c_str(); }

int md_tree_validate(const md_tree* t, int K, const int32_t* k_per_head) { return expand_tree(t, K, k_per_head, nullptr); }



static bool known_kind(int kind) {
    return kind == MD_HEADS_MEDUSA || kind == MD_HEADS_HYDRA || kind == MD_HEADS_MEDUSA_SHARED;
}

int64_t md_heads_weight_bytes(int kind, int dt, int d, int V, int K) {
    if (!known_kind(kind) || (dt != MD_F32 && dt != MD_BF16) || d < 1 || V < 1 || K < 1) return -1;
    const int64_t din = kind == MD_HEADS_HYDRA ? 2LL * d : (int64_t)d;
    const int64_t residual = (int64_t)d * din + d, projection = (int64_t)V * d;
    const int64_t params = kind == MD_HEADS_MEDUSA_SHARED ? K * residual + projection : K * (residual + projection);
    return params * (dt == MD_F32 ? 4 : 2);
}

int md_heads_fused(int kind, int dt, int M, int d, int K) {
    if (!known_kind(kind) || K < 1 || K > MD_MAX_HEADS) return 0;
    return kind == MD_HEADS_MEDUSA && heads_fused_applicable(dt, M, d, d, 0, K) ? 1 : 0;
}

float md_certified_rounding_allowance(int d) { return d > 0 ? cert_rounding_allowance(d) : -1.f; }

size_t md_heads_workspace_bytes(int kind, int dt, int M, int d, int V, int K, int kmax) {
    if (M <= 0 || d <= 0 || V <= 0 || K <= 0 || kmax <= 0) return 0;
    if (kind == MD_HEADS_HYDRA) {
        // any level has at most 63 parents per request; size for every row count up to that
        size_t need = 0;
        for (int rows = M; rows <= M * (MD_MAX_NODES - 1); rows += M) {
            const size_t b = heads_ws_bound(dt, rows, d, 2 * d, V, 1, kmax, 0);
            if (b > need) need = b;
        }
        return need;
    }
    return heads_ws_bound(dt, M, d, d, V, K, kmax, kind == MD_HEADS_MEDUSA_SHARED);
}

int md_medusa_heads(int kind, int dt, int M, int d, int V, int K, const int32_t* k_per_head, int level,
                    const md_tree* tree, const void* h, const void* W, const void* b, const void* U, const void* U_op,
                    const float* U_norms, const void* W_op, const void* E, const int32_t* root_tok,
                    const int32_t* tree_tok, int32_t* topk_idx, float* topk_val, float* h_res, void* ws,
                    size_t ws_bytes, void* stream) {
    if (!known_kind(kind)) return fail(MD_EINVAL, "kind = %d", kind);
    if (check_dt(dt)) return MD_EINVAL;
    if (U_op && dt != MD_BF16) return fail(MD_EINVAL, "an operand-order copy of U exists for bf16 only");
    if (U_norms && dt != MD_BF16) return fail(MD_EINVAL, "tile norms of U exist for bf16 only");
    if (W_op && dt != MD_BF16) return fail(MD_EINVAL, "an operand-order copy of W exists for bf16 only");
    if (M < 0) return fail(MD_EINVAL, "M = %d", M);
    if (K < 1 || K > MD_MAX_HEADS) return fail(MD_EINVAL, "K = %d heads (1..8 supported)", K);
    if (!k_per_head) return fail(MD_EINVAL, "k_per_head is NULL");
    int kmax = 0;
    for (int i = 0; i < K; ++i) {
        if (k_per_head[i] < 1 || k_per_head[i] > MD_MAX_TOPK)
            return fail(MD_EINVAL, "k_per_head[%d] = %d (1..16 supported)", i, k_per_head[i]);
        if (k_per_head[i] > kmax) kmax = k_per_head[i];
    }
    if (d < 8 || d % 8) return fail(MD_EUNSUPPORTED, "d = %d (a positive multiple of 8 is required)", d);
    const int din = kind == MD_HEADS_HYDRA ? 2 * d : d;
    if ((size_t)din * 4 > 160 * 1024) return fail(MD_EUNSUPPORTED, "input width %d exceeds one LDS row buffer", din);
    if (V < kmax) return fail(MD_EINVAL, "V = %d is smaller than the widest top-k %d", V, kmax);
    if (M == 0) return MD_OK;
    if (!h || !W || !U || !topk_idx || !topk_val || !ws) return fail(MD_EINVAL, "a required pointer is NULL");

    HeadsArgs a;
    memset(&a, 0, sizeof(a));
    DevTree dt_tree;
    const DevTree* tp = nullptr;
    a.kind = kind == MD_HEADS_HYDRA ? 1 : 0;
    a.shared_u = kind == MD_HEADS_MEDUSA_SHARED;
    a.dt = dt;
    a.d = d;
    a.din = din;
    a.V = V;
    a.kmax = kmax;
    a.level = level;
    a.h = h;
    a.W = W;
    a.b = b;
    a.U = U;
    a.U_op = U_op;
    a.U_norms = U_norms;
    a.W_op = W_op;
    a.E = E;
    a.root_tok = root_tok;
    a.tree_tok = tree_tok;
    a.topk_idx = topk_idx;
    a.topk_val = topk_val;
    a.h_res = h_res;
    a.ws = ws;
    size_t need;
    if (kind != MD_HEADS_HYDRA) {
        if (level != 0) return fail(MD_EINVAL, "Medusa heads take level 0 (got %d)", level);
        a.M = M;
        a.B = M;
        a.nh = K;
        a.head0 = 0;
        for (int i = 0; i < K; ++i) a.kk[i] = k_per_head[i];
        need = heads_ws_bytes(dt, M, d, d, V, K, kmax, a.shared_u, U_op != nullptr);
    } else {
        if (level < 1 || level > K) return fail(MD_EINVAL, "Hydra level %d outside 1..%d", level, K);
        int rc = expand_tree(tree, K, k_per_head, &dt_tree);
        if (rc) return rc;
        if (!E || !root_tok) return fail(MD_EINVAL, "Hydra heads need E and root_tok");
        if (level >= 2 && !tree_tok) return fail(MD_EINVAL, "Hydra level %d needs tree_tok", level);
        const int P = dt_tree.level_off[level + 1] - dt_tree.level_off[level];
        a.M = M * P;
        a.B = M;
        a.nh = 1;
        a.head0 = level - 1;
        a.kk[0] = k_per_head[level - 1];
        tp = &dt_tree;
        if (P == 0) return MD_OK;  // nothing at this depth
        need = heads_ws_bytes(dt, a.M, d, din, V, 1, kmax, 0, U_op != nullptr);
    }
    if (ws_bytes < need) return fail(MD_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    a.spin_res = g_spin_res;
    a.spin_lists = g_spin_lists;
    return hip_status(heads_launch(a, tp, (hipStream_t)stream, g_ev0, g_ev1), "md_medusa_heads");
}

int md_tree_build(const md_tree* tree, int kind, int B, int M, int K, int kmax, int level, const int32_t* topk_idx,
                  const int32_t* src_row, const int32_t* root_tok, const int32_t* lens, int32_t* tree_tok,
                  int32_t* tree_pos, void* stream) {
    DevTree t;
    int rc = expand_tree(tree, K, nullptr, &t);
    if (rc) return rc;
    if (!known_kind(kind)) return fail(MD_EINVAL, "kind = %d", kind);
    if (B < 0 || kmax < 1 || kmax > MD_MAX_TOPK) return fail(MD_EINVAL, "B = %d, kmax = %d", B, kmax);
    for (int n = 1; n < t.n; ++n)
        if (t.rank[n] >= kmax) return fail(MD_EINVAL, "node %d: rank %d but lists hold %d", n, t.rank[n], kmax);
    if (kind != MD_HEADS_HYDRA) {
        if (level != 0) return fail(MD_EINVAL, "Medusa trees build all levels at once (level 0)");
        if (M < 1) return fail(MD_EINVAL, "M = %d", M);
        if (B > 0 && !src_row) return fail(MD_EINVAL, "src_row is NULL");
    } else {
        if (level < 1 || level > K) return fail(MD_EINVAL, "Hydra level %d outside 1..%d", level, K);
        if (level > t.max_depth) return MD_OK;
    }
    if (B == 0) return MD_OK;
    if (!topk_idx || !root_tok || !lens || !tree_tok || !tree_pos) return fail(MD_EINVAL, "a required pointer is NULL");
    return hip_status(tree_build_launch(t, kind == MD_HEADS_HYDRA ? 1 : 0, B, M, K, kmax, level, topk_idx, src_row, root_tok, lens, tree_tok,
                                        tree_pos, (hipStream_t)stream),
                      "md_tree_build");
}

size_t md_attention_workspace_bytes(int dt, int B, int N, int Hq, int Hkv, int hd, int max_len) {
    if (B <= 0 || N <= 0 || Hq <= 0 || Hkv <= 0 || hd <= 0 || max_len < 0 || Hq % Hkv) return 0;
    return attention_ws_bytes(dt, B, N, Hq, Hkv, hd, max_len);
}

int md_tree_attention(const md_tree* tree, int dt, int B, int Hq, int Hkv, int hd, int Lcap, int max_len,
                      const void* q, const void* Kc, const void* Vc, const int32_t* lens, float scale, void* out,
                      void* ws, size_t ws_bytes, void* stream) {
    DevTree t;
    int rc = expand_tree(tree, MD_MAX_HEADS, nullptr, &t);
    if (rc) return rc;
    if (check_dt(dt)) return MD_EINVAL;
    if (B < 0 || Hq < 1 || Hkv < 1) return fail(MD_EINVAL, "B = %d, Hq = %d, Hkv = %d", B, Hq, Hkv);
    if (Hq % Hkv) return fail(MD_EINVAL, "Hq = %d is not a multiple of Hkv = %d", Hq, Hkv);
    if (hd != 64 && hd != 128) return fail(MD_EUNSUPPORTED, "head_dim %d (64 or 128 supported)", hd);
    if (max_len < 0) return fail(MD_EINVAL, "max_len = %d", max_len);
    if ((int64_t)max_len + t.n > Lcap) return fail(MD_ERANGE, "max_len %d + %d nodes exceeds Lcap %d", max_len, t.n, Lcap);
    if (B == 0) return MD_OK;
    if (!q || !Kc || !Vc || !lens || !out || !ws) return fail(MD_EINVAL, "a required pointer is NULL");
    const size_t need = attention_ws_bytes(dt, B, t.n, Hq, Hkv, hd, max_len);
    if (ws_bytes < need) return fail(MD_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    return hip_status(attention_launch(t, dt, B, Hq, Hkv, hd, Lcap, max_len, q, Kc, Vc, lens, scale, out, ws,
                                       (hipStream_t)stream),
                      "md_tree_attention");
}

int md_tree_attention_noalloc(const md_tree* tree, int dt, int B, int Hq, int Hkv, int hd, int Lcap, int max_len,
                              const void* q, const void* Kc, const void* Vc, const int32_t* lens, float scale,
                              void* out, void* stream) {
    DevTree t;
    int rc = expand_tree(tree, MD_MAX_HEADS, nullptr, &t);
    if (rc) return rc;
    if (check_dt(dt)) return MD_EINVAL;
    if (B < 0 || Hq < 1 || Hkv < 1) return fail(MD_EINVAL, "B = %d, Hq = %d, Hkv = %d", B, Hq, Hkv);
    if (Hq % Hkv) return fail(MD_EINVAL, "Hq = %d is not a multiple of Hkv = %d", Hq, Hkv);
    if (hd != 64 && hd != 128) return fail(MD_EUNSUPPORTED, "head_dim %d (64 or 128 supported)", hd);
    if (max_len < 0) return fail(MD_EINVAL, "max_len = %d", max_len);
    if ((int64_t)max_len + t.n > Lcap) return fail(MD_ERANGE, "max_len %d + %d nodes exceeds Lcap %d", max_len, t.n, Lcap);
    if (B == 0) return MD_OK;
    if (!q || !Kc || !Vc || !lens || !out) return fail(MD_EINVAL, "a required pointer is NULL");
    const size_t need = attention_ws_bytes(dt, B, t.n, Hq, Hkv, hd, max_len);
    if (need > kAttnScratchBytes)
        return fail(MD_EWORKSPACE, "these sizes need %zu bytes of scratch; the library's static scratch holds %zu",
                    need, kAttnScratchBytes);
    void* ws = nullptr;
    rc = hip_status(attention_scratch(&ws), "md_tree_attention_noalloc (scratch address)");
    if (rc) return rc;
    return hip_status(attention_launch(t, dt, B, Hq, Hkv, hd, Lcap, max_len, q, Kc, Vc, lens, scale, out, ws,
                                       (hipStream_t)stream),
                      "md_tree_attention_noalloc");
}

size_t md_tree_attention_noalloc_max_bytes(void) { return kAttnScratchBytes; }

size_t md_accept_workspace_bytes(int B, int N, int V) {
    if (B <= 0 || N <= 0 || V <= 0) return 0;
    return accept_ws_bytes(B, N, V);
}

int md_tree_accept(const md_tree* tree, int dt, int B, int K, int V, int Hkv, int hd, int Lcap, const float* logits,
                   const int32_t* tree_tok, void* Kc, void* Vc, int32_t* lens, int32_t* accept_len, int32_t* path,
                   int32_t* next_tok, int32_t* compact_src, void* ws, size_t ws_bytes, void* stream) {
    DevTree t;
    int rc = expand_tree(tree, K, nullptr, &t);
    if (rc) return rc;
    if (check_dt(dt)) return MD_EINVAL;
    if (B < 0 || V < 1 || Hkv < 1 || hd < 1) return fail(MD_EINVAL, "B = %d, V = %d, Hkv = %d, hd = %d", B, V, Hkv, hd);
    if (hd > 256) return fail(MD_EUNSUPPORTED, "head_dim %d (at most 256)", hd);
    if (Lcap < t.n) return fail(MD_ERANGE, "Lcap %d is smaller than the tree (%d nodes)", Lcap, t.n);
    if (B == 0) return MD_OK;
    if (!logits || !tree_tok || !Kc || !Vc || !lens || !accept_len || !path || !next_tok || !compact_src || !ws)
        return fail(MD_EINVAL, "a required pointer is NULL");
    const size_t need = accept_ws_bytes(B, t.n, V);
    if (ws_bytes < need) return fail(MD_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    return hip_status(accept_launch(t, dt, B, K, V, Hkv, hd, Lcap, logits, tree_tok, Kc, Vc, lens, accept_len, path,
                                    next_tok, compact_src, ws, (hipStream_t)stream),
                      "md_tree_accept");
}

size_t md_target_argmax_workspace_bytes(int dt, int R, int d, int V) {
    if ((dt != MD_F32 && dt != MD_BF16) || R <= 0 || d <= 0 || V <= 0) return 0;
    return target_argmax_ws_bound(dt, R, d, V);
}

int md_target_argmax(int dt, int R, int d, int V, const void* H, const void* Wt, const void* Wt_op, int32_t* tok,
                     float* val, void* ws, size_t ws_bytes, void* stream) {
    if (check_dt(dt)) return MD_EINVAL;
    if (Wt_op && dt != MD_BF16) return fail(MD_EINVAL, "an operand-order copy of Wt exists for bf16 only");
    if (R < 0 || V < 1) return fail(MD_EINVAL, "R = %d, V = %d", R, V);
    if (d < 8 || d % 8) return fail(MD_EUNSUPPORTED, "d = %d (a positive multiple of 8 is required)", d);
    if ((size_t)d * 4 > 160 * 1024) return fail(MD_EUNSUPPORTED, "width %d exceeds one LDS row buffer", d);
    if (R == 0) return MD_OK;
    if (!H || !Wt || !tok || !ws) return fail(MD_EINVAL, "a required pointer is NULL");
    const size_t need = target_argmax_ws_bound(dt, R, d, V);
    if (ws_bytes < need) return fail(MD_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    return hip_status(target_argmax_launch(dt, R, d, V, H, Wt, Wt_op, tok, val, ws, (hipStream_t)stream),
                      "md_target_argmax");
}

size_t md_operand_order_bytes(int nmat, int rows, int cols) {
    if (nmat < 1 || rows < 1 || cols < 32 || cols % 32) return 0;
    return operand_order_bytes(nmat, rows, cols);
}

int md_operand_order(int nmat, int rows, int cols, const void* src, void* dst, void* stream) {
    if (nmat < 1 || rows < 1) return fail(MD_EINVAL, "nmat = %d, rows = %d", nmat, rows);
    if (cols < 32 || cols % 32) return fail(MD_EUNSUPPORTED, "cols = %d (a positive multiple of 32 is required)", cols);
    if (!src || !dst) return fail(MD_EINVAL, "a required pointer is NULL");
    return hip_status(operand_order_launch(nmat, rows, cols, src, dst, (hipStream_t)stream), "md_operand_order");
}

size_t md_vocab_tile_norms_bytes(int nmat, int V) {
    if (nmat < 1 || V < 1) return 0;
    return (size_t)nmat * vocab_tiles(V) * sizeof(float);
}

int md_vocab_tile_norms(int nmat, int V, int d, const void* U, float* norms, void* stream) {
    if (nmat < 1 || V < 1) return fail(MD_EINVAL, "nmat = %d, V = %d", nmat, V);
    if (d < 8 || d % 8) return fail(MD_EUNSUPPORTED, "d = %d (a positive multiple of 8 is required)", d);
    if (!U || !norms) return fail(MD_EINVAL, "a required pointer is NULL");
    return hip_status(vocab_tile_norms_launch(U, nmat, V, d, norms, (hipStream_t)stream), "md_vocab_tile_norms");
}

int md_tree_accept_tokens(const md_tree* tree, int dt, int B, int K, int Hkv, int hd, int Lcap,
                          const int32_t* target_tok, const int32_t* tree_tok, void* Kc, void* Vc, int32_t* lens,
                          int32_t* accept_len, int32_t* path, int32_t* next_tok, int32_t* compact_src, void* stream) {
    DevTree t;
    int rc = expand_tree(tree, K, nullptr, &t);
    if (rc) return rc;
    if (check_dt(dt)) return MD_EINVAL;
    if (B < 0 || Hkv < 1 || hd < 1) return fail(MD_EINVAL, "B = %d, Hkv = %d, hd = %d", B, Hkv, hd);
    if (hd > 256) return fail(MD_EUNSUPPORTED, "head_dim %d (at most 256)", hd);
    if (Lcap < t.n) return fail(MD_ERANGE, "Lcap %d is smaller than the tree (%d nodes)", Lcap, t.n);
    if (B == 0) return MD_OK;
    if (!target_tok || !tree_tok || !Kc || !Vc || !lens || !accept_len || !path || !next_tok || !compact_src)
        return fail(MD_EINVAL, "a required pointer is NULL");
    return hip_status(accept_tokens_launch(t, dt, B, K, Hkv, hd, Lcap, target_tok, tree_tok, Kc, Vc, lens, accept_len,
                                           path, next_tok, compact_src, (hipStream_t)stream),
                      "md_tree_accept_tokens");
}

static bool good_temperature(float T) { return T > 0.0f && T <= 3.0e38f; }

size_t md_heads_logits_workspace_bytes(int kind, int M, int d, int K) {
    if ((kind != MD_HEADS_MEDUSA && kind != MD_HEADS_MEDUSA_SHARED) || M <= 0 || d <= 0 || K <= 0) return 0;
    return heads_logits_ws_bytes(M, d, K);
}

int md_medusa_heads_logits(int kind, int dt, int M, int d, int V, int K, const void* h, const void* W, const void* b,
                           const void* U, float* logits, float* h_res, void* ws, size_t ws_bytes, void* stream) {
    if (kind != MD_HEADS_MEDUSA && kind != MD_HEADS_MEDUSA_SHARED)
        return fail(MD_EINVAL, "kind = %d (Medusa kinds only)", kind);
    if (check_dt(dt)) return MD_EINVAL;
    if (M < 0 || V < 1) return fail(MD_EINVAL, "M = %d, V = %d", M, V);
    if (K < 1 || K > MD_MAX_HEADS) return fail(MD_EINVAL, "K = %d heads (1..8 supported)", K);
    if (d < 8 || d % 8) return fail(MD_EUNSUPPORTED, "d = %d (a positive multiple of 8 is required)", d);
    if ((size_t)d * 4 > 160 * 1024) return fail(MD_EUNSUPPORTED, "input width %d exceeds one LDS row buffer", d);
    if (M == 0) return MD_OK;
    if (!h || !W || !U || !logits || !ws) return fail(MD_EINVAL, "a required pointer is NULL");
    const size_t need = heads_logits_ws_bytes(M, d, K);
    if (ws_bytes < need) return fail(MD_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    HeadsArgs a;
    memset(&a, 0, sizeof(a));
    a.spin_res = a.spin_lists = -1;  // the single-launch kernel does not run here
    a.kind = 0;
    a.shared_u = kind == MD_HEADS_MEDUSA_SHARED;
    a.dt = dt;
    a.M = M;
    a.B = M;
    a.d = d;
    a.din = d;
    a.V = V;
    a.nh = K;
    a.kmax = 1;
    for (int i = 0; i < K; ++i) a.kk[i] = 1;
    a.h = h;
    a.W = W;
    a.b = b;
    a.U = U;
    a.h_res = h_res;
    a.ws = ws;
    a.logits = logits;
    a.logits_k = K;
    return hip_status(heads_launch(a, nullptr, (hipStream_t)stream, g_ev0, g_ev1), "md_medusa_heads_logits");
}

size_t md_draft_sample_workspace_bytes(int M, int K, int V, int kmax) {
    if (M <= 0 || K <= 0 || K > MD_MAX_HEADS || V <= 0 || kmax <= 0 || kmax > MD_MAX_TOPK) return 0;
    return draft_sample_ws_bytes(M, K, V, kmax);
}

int md_draft_sample(int M, int K, int V, const int32_t* k_per_head, float temperature, const float* logits,
                    const uint32_t* words, int32_t* tok, float* lse, void* ws, size_t ws_bytes, void* stream) {
    if (M < 0 || V < 1) return fail(MD_EINVAL, "M = %d, V = %d", M, V);
    if (K < 1 || K > MD_MAX_HEADS) return fail(MD_EINVAL, "K = %d heads (1..8 supported)", K);
    if (!k_per_head) return fail(MD_EINVAL, "k_per_head is NULL");
    int kk[MD_MAX_HEADS], kmax = 0;
    for (int i = 0; i < K; ++i) {
        if (k_per_head[i] < 1 || k_per_head[i] > MD_MAX_TOPK)
            return fail(MD_EINVAL, "k_per_head[%d] = %d (1..16 supported)", i, k_per_head[i]);
        kk[i] = k_per_head[i];
        if (kk[i] > kmax) kmax = kk[i];
    }
    if (V < kmax) return fail(MD_EINVAL, "V = %d is smaller than the widest draw %d", V, kmax);
    if (!good_temperature(temperature)) return fail(MD_EINVAL, "temperature %g (positive and finite)", (double)temperature);
    if (M == 0) return MD_OK;
    if (!logits || !words || !tok || !lse || !ws) return fail(MD_EINVAL, "a required pointer is NULL");
    const size_t need = draft_sample_ws_bytes(M, K, V, kmax);
    if (ws_bytes < need) return fail(MD_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    return hip_status(draft_sample_launch(M, K, V, kk, kmax, temperature, logits, words, tok, lse, ws,
                                          (hipStream_t)stream),
                      "md_draft_sample");
}

// the checks md_tree_accept_tokens makes, shared by the sampled verifiers
static int check_accept_args(const DevTree& t, int dt, int B, int V, int Hkv, int hd, int Lcap) {
    if (check_dt(dt)) return MD_EINVAL;
    if (B < 0 || V < 1 || Hkv < 1 || hd < 1) return fail(MD_EINVAL, "B = %d, V = %d, Hkv = %d, hd = %d", B, V, Hkv, hd);
    if (hd > 256) return fail(MD_EUNSUPPORTED, "head_dim %d (at most 256)", hd);
    if (Lcap < t.n) return fail(MD_ERANGE, "Lcap %d is smaller than the tree (%d nodes)", Lcap, t.n);
    return MD_OK;
}

size_t md_verify_sampled_workspace_bytes(int B, int N) {
    if (B <= 0 || N <= 0 || N > MD_MAX_NODES) return 0;
    return verify_sampled_ws_bytes(B, N);
}

int md_tree_verify_sampled(const md_tree* tree, int dt, int B, int K, int V, int Hkv, int hd, int Lcap,
                           float temperature, const float* target_logits, const float* head_logits,
                           const float* head_lse, const int32_t* tree_tok, const uint32_t* u_words,
                           const uint32_t* g_words, void* Kc, void* Vc, int32_t* lens, int32_t* accept_len,
                           int32_t* path, int32_t* next_tok, int32_t* compact_src, void* ws, size_t ws_bytes,
                           void* stream) {
    DevTree t;
    int rc = expand_tree(tree, K, nullptr, &t);
    if (rc) return rc;
    rc = check_accept_args(t, dt, B, V, Hkv, hd, Lcap);
    if (rc) return rc;
    if (!good_temperature(temperature)) return fail(MD_EINVAL, "temperature %g (positive and finite)", (double)temperature);
    if (B == 0) return MD_OK;
    if (!target_logits || !head_logits || !head_lse || !tree_tok || !u_words || !g_words || !Kc || !Vc || !lens ||
        !accept_len || !path || !next_tok || !compact_src || !ws)
        return fail(MD_EINVAL, "a required pointer is NULL");
    const size_t need = verify_sampled_ws_bytes(B, t.n);
    if (ws_bytes < need) return fail(MD_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    return hip_status(verify_sampled_launch(t, dt, B, K, V, Hkv, hd, Lcap, temperature, target_logits, head_logits,
                                            head_lse, tree_tok, u_words, g_words, Kc, Vc, lens, accept_len, path,
                                            next_tok, compact_src, ws, (hipStream_t)stream),
                      "md_tree_verify_sampled");
}

size_t md_accept_typical_workspace_bytes(int B, int N) {
    if (B <= 0 || N <= 0 || N > MD_MAX_NODES) return 0;
    return accept_typical_ws_bytes(B, N);
}

int md_tree_accept_typical(const md_tree* tree, int dt, int B, int K, int V, int Hkv, int hd, int Lcap,
                           float temperature, float eps, float delta, const float* target_logits,
                           const int32_t* tree_tok, const uint32_t* g_words, void* Kc, void* Vc, int32_t* lens,
                           int32_t* accept_len, int32_t* path, int32_t* next_tok, int32_t* compact_src, void* ws,
                           size_t ws_bytes, void* stream) {
    DevTree t;
    int rc = expand_tree(tree, K, nullptr, &t);
    if (rc) return rc;
    rc = check_accept_args(t, dt, B, V, Hkv, hd, Lcap);
    if (rc) return rc;
    if (!good_temperature(temperature)) return fail(MD_EINVAL, "temperature %g (positive and finite)", (double)temperature);
    if (!(eps >= 0.0f && eps <= 3.0e38f) || !(delta >= 0.0f && delta <= 3.0e38f))
        return fail(MD_EINVAL, "eps = %g, delta = %g (non-negative and finite)", (double)eps, (double)delta);
    if (B == 0) return MD_OK;
    if (!target_logits || !tree_tok || !g_words || !Kc || !Vc || !lens || !accept_len || !path || !next_tok ||
        !compact_src || !ws)
        return fail(MD_EINVAL, "a required pointer is NULL");
    const size_t need = accept_typical_ws_bytes(B, t.n);
    if (ws_bytes < need) return fail(MD_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    return hip_status(accept_typical_launch(t, dt, B, K, V, Hkv, hd, Lcap, temperature, eps, delta, target_logits,
                                            tree_tok, g_words, Kc, Vc, lens, accept_len, path, next_tok, compact_src,
                                            ws, (hipStream_t)stream),
                      "md_tree_accept_typical");
}

int md_hbm_read_probe_blocks(void) { return probe_blocks(); }

int md_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    if (!buf || !sink) return fail(MD_EINVAL, "a required pointer is NULL");
    if (bytes == 0 || bytes % 16) return fail(MD_EINVAL, "bytes = %zu (a positive multiple of 16)", bytes);
    return hip_status(probe_launch(buf, bytes, sink, (hipStream_t)stream), "md_hbm_read_probe");
}

int md_set_wait_limits(int residual_polls, int list_polls) {
    if (residual_polls < -1 || list_polls < -1)
        return fail(MD_EINVAL, "poll limits %d, %d (-1 or more)", residual_polls, list_polls);
    g_spin_res = residual_polls;
    g_spin_lists = list_polls;
    return MD_OK;
}

int md_set_vocab_timing_events(void* start, void* stop) {
    if ((start == nullptr) != (stop == nullptr)) return fail(MD_EINVAL, "pass two events or none");
    g_ev0 = (hipEvent_t)start;
    g_ev1 = (hipEvent_t)stop;
    return MD_OK;
}

}  // extern "C"
