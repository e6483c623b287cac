// Sampled decoding on the tree: drafts drawn from the heads' distributions,
// verification by rejection sampling, and typical acceptance.
//
// "Medusa heads versus separate draft model", section "Training": with
// sampling at a temperature, keeping the target's distribution exactly
// takes rejection sampling with the heads' probabilities; Medusa's "typical
// acceptance" takes more drafts but does not keep it. The pages give neither
// procedure on a tree. Readings taken here:
//
// * draft distribution of head i: q_i = softmax(l_i / T); the target's at
//   node n: p_n = softmax(target_logits[n] / T);
// * head i's draft tokens are k_i distinct tokens drawn from q_i without
//   replacement, in draw order: the k_i largest of l_i / T + Gumbel noise;
// * verification walks down from the root. At a node the children are tried
//   in rank order: child x is accepted with probability min(1, p(x) / q(x));
//   on rejection p <- normalise(max(0, p - q)) and x leaves q (q is
//   renormalised), the rule for candidates drawn without replacement. An
//   accepted child becomes the node; with every child rejected, or at a
//   leaf, the step's last token is drawn from the current p;
// * typical acceptance: node n matches when its parent's p gives tok(n) more
//   than min(eps, delta exp(-H(p))), H the entropy; the deepest node whose
//   root path matches (lowest index among equals) ends the step, and the
//   last token is drawn from that node's p;
// * a tree token outside [0, V) is never accepted and changes nothing.
//
// The walk never forms the residual vectors. A rejected x had p(x) < q(x)
// (else the test accepts: u < 1), so its residual entry is 0 and stays 0;
// by induction the residual after j rejections is, unnormalised,
// R_j(y) = max(0, p(y) - c_j q(y)) for every y, with c_1 = 0 and
// c_{j+1} = c_j + M_j / S_j, where M_j = sum_y R_j(y) and S_j = 1 - the
// q-mass of the rejected tokens. Each rejection costs one reduction over the
// vocabulary (M_{j+1}); the acceptance ratio of candidate j is
// (R_j(x) / M_j) / (q(x) / S_j). The final draw is a Gumbel-max over
// log R(y), which needs no normalisation.
//
// Random numbers arrive as 32-bit words: u = (w / 2^9 + 1/2) 2^-23 lies in
// (0, 1) and is exact in float; Gumbel noise is -log(-log u).
#include <math.h>

#include "md_internal.h"

namespace {

constexpr int BLOCK = 256;
constexpr int NWAVE = BLOCK / MD_WAVE;
constexpr int KM = 16;     // longest draft list
constexpr int WALK = 1024;  // threads of a walk block: 16 waves stream one request's vocabulary rows
constexpr int WWAVES = WALK / MD_WAVE;
constexpr int kDraftBlocks = 1024;

__device__ __forceinline__ bool above(float v, int i, float w, int j) { return v > w || (v == w && i < j); }

__device__ __forceinline__ float unit_f(uint32_t w) { return ((float)(w >> 9) + 0.5f) * 0x1p-23f; }

__device__ __forceinline__ float gumbel_f(uint32_t w) { return -logf(-logf(unit_f(w))); }

// Online log-sum-exp state: m the largest term, s = sum exp(z - m).
__device__ __forceinline__ void lse_add(float& m, float& s, float z) {
    if (z > m) {
        s = s * __expf(m - z) + 1.0f;
        m = z;
    } else {
        s += __expf(z - m);
    }
}

template <int NW>
__device__ double block_sum(double x, double* sh) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, MD_WAVE);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) sh[w] = x;
    __syncthreads();
    double t = 0.0;
#pragma unroll
    for (int i = 0; i < NW; ++i) t += sh[i];  // same order in every thread
    __syncthreads();
    return t;
}

// Combine per-thread (m, s) log-sum-exp states; every thread gets log sum exp.
template <int NW>
__device__ double block_lse(float m, float s, float* shm, double* shs) {
    float bm = m;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) bm = fmaxf(bm, __shfl_xor(bm, o, MD_WAVE));
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) shm[w] = bm;
    __syncthreads();
    float M = shm[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) M = fmaxf(M, shm[i]);
    const double part = s > 0.0f ? (double)s * exp((double)m - (double)M) : 0.0;
    const double S = block_sum<NW>(part, shs);
    return (double)M + log(S);
}

// Block argmax over (value desc, index asc); every thread gets the winner.
template <int NW>
__device__ void block_argmax(float& v, int& i, float* shv, int* shi) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(v, o, MD_WAVE);
        const int oi = __shfl_xor(i, o, MD_WAVE);
        if (above(ov, oi, v, i)) {
            v = ov;
            i = oi;
        }
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        shv[w] = v;
        shi[w] = i;
    }
    __syncthreads();
    v = shv[0];
    i = shi[0];
#pragma unroll
    for (int k = 1; k < NW; ++k)
        if (above(shv[k], shi[k], v, i)) {
            v = shv[k];
            i = shi[k];
        }
    __syncthreads();
}

// ------------------------------------------------------------ draft sample

struct KS {
    int v[8];
};

// Block (row-head rh = m K + h, vocabulary chunk ch): the chunk's k best
// perturbed values l / T + G as one sorted list, and its log-sum-exp.
// Lists are laid out [h][m][chunk][kmax] for the k-way merge.
__global__ __launch_bounds__(BLOCK) void k_draft_part(const float* __restrict__ logits,
                                                      const uint32_t* __restrict__ words, int M, int K, int V,
                                                      float invT, int chunks, KS ks, int kmax,
                                                      float* __restrict__ part_v, int* __restrict__ part_i,
                                                      float* __restrict__ part_lse) {
    __shared__ float shv[NWAVE], shm[NWAVE];
    __shared__ int shi[NWAVE];
    __shared__ double shs[NWAVE];
    __shared__ float out_v[KM];
    __shared__ int out_i[KM];
    const int rh = blockIdx.x / chunks, ch = blockIdx.x - rh * chunks;
    const int m = rh / K, h = rh - m * K;
    const int k = ks.v[h];
    const int tid = threadIdx.x;
    const int a = (int)((int64_t)V * ch / chunks), e = (int)((int64_t)V * (ch + 1) / chunks);
    const float* lg = logits + (int64_t)rh * V;
    const uint32_t* wd = words + (int64_t)rh * V;
    float v[KM];
    int ix[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
        v[j] = -INFINITY;
        ix[j] = INT_MAX;
    }
    float lm = -INFINITY, ls = 0.0f;
    for (int y = a + tid; y < e; y += BLOCK) {
        const float z = lg[y] * invT;
        lse_add(lm, ls, z);
        const float s = z + gumbel_f(wd[y]);
        if (!above(s, y, v[KM - 1], ix[KM - 1])) continue;
#pragma unroll
        for (int q = KM - 1; q >= 0; --q) {  // insertion; v[q - 1] is read before it moves
            if (!above(s, y, v[q], ix[q])) continue;
            if (q > 0 && above(s, y, v[q - 1], ix[q - 1])) {
                v[q] = v[q - 1];
                ix[q] = ix[q - 1];
            } else {
                v[q] = s;
                ix[q] = y;
            }
        }
    }
    const double lse = block_lse<NWAVE>(lm, ls, shm, shs);
    // k rounds of a block argmax over the thread lists' heads
    for (int r = 0; r < k; ++r) {
        float bv = v[0];
        int bi = ix[0];
        block_argmax<NWAVE>(bv, bi, shv, shi);
        if (tid == 0) {
            out_v[r] = bv;
            out_i[r] = bi;
        }
        if (bi != INT_MAX && ix[0] == bi) {  // indices are unique: the owner pops its head
#pragma unroll
            for (int j = 0; j + 1 < KM; ++j) {
                v[j] = v[j + 1];
                ix[j] = ix[j + 1];
            }
            v[KM - 1] = -INFINITY;
            ix[KM - 1] = INT_MAX;
        }
    }
    __syncthreads();
    const int64_t base = (((int64_t)h * M + m) * chunks + ch) * kmax;
    if (tid < kmax) {
        part_v[base + tid] = tid < k ? out_v[tid] : -INFINITY;
        part_i[base + tid] = tid < k ? out_i[tid] : INT_MAX;
    }
    if (tid == 0) part_lse[(int64_t)rh * chunks + ch] = (float)lse;  // -inf for an empty chunk
}

__global__ void k_lse_merge(const float* __restrict__ part_lse, int rows, int chunks, float* __restrict__ lse) {
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= rows) return;
    const float* pl = part_lse + (int64_t)r * chunks;
    double M = -INFINITY;
    for (int c = 0; c < chunks; ++c) M = fmax(M, (double)pl[c]);
    double S = 0.0;
    for (int c = 0; c < chunks; ++c)
        if (pl[c] > -INFINITY) S += exp((double)pl[c] - M);
    lse[r] = (float)(M + log(S));
}

int draft_chunks(int rows, int V) {
    int c = (kDraftBlocks + rows - 1) / rows;
    const int max_c = (V + BLOCK - 1) / BLOCK;  // at least a thread's worth each
    if (c > max_c) c = max_c;
    return c < 1 ? 1 : c;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ------------------------------------------------------------- the walk

__device__ __forceinline__ int first_child(const DevTree& t, int node) {
    for (int n = node + 1; n < t.n; ++n)
        if (t.parent[n] == node) return n;
    return -1;
}

__device__ __forceinline__ int next_sibling(const DevTree& t, int n) {
    for (int s = n + 1; s < t.n; ++s)
        if (t.parent[s] == t.parent[n]) return s;
    return -1;
}

// One block per request. Every thread runs the same walk on the same
// scalars; the vocabulary sweeps are block reductions.
__global__ __launch_bounds__(WALK) void k_walk_sampled(DevTree t, int K, int V, float invT,
                                                       const float* __restrict__ target_logits,
                                                       const float* __restrict__ head_logits,
                                                       const float* __restrict__ head_lse,
                                                       const int32_t* __restrict__ tree_tok,
                                                       const uint32_t* __restrict__ u_words,
                                                       const uint32_t* __restrict__ g_words,
                                                       int32_t* __restrict__ chosen) {
    __shared__ float shv[WWAVES], shm[WWAVES];
    __shared__ int shi[WWAVES];
    __shared__ double shs[WWAVES];
    const int b = blockIdx.x, N = t.n, tid = threadIdx.x;
    if (tid < N) chosen[(int64_t)b * N + tid] = -1;
    const uint32_t* gw = g_words + (int64_t)b * V;
    int node = 0;
    while (true) {
        const float* lt = target_logits + ((int64_t)b * N + node) * V;
        const int c0 = first_child(t, node);
        double c = 0.0;  // residual R(y) = max(0, p(y) - c q(y)); the sweeps use it in float
        const float* lh = nullptr;
        float lse_t = 0.0f, lse_h = 0.0f;
        int next = -1;
        if (c0 >= 0) {
            float lm = -INFINITY, ls = 0.0f;
            for (int y = tid; y < V; y += WALK) lse_add(lm, ls, lt[y] * invT);
            lse_t = (float)block_lse<WWAVES>(lm, ls, shm, shs);
            const int hd = t.depth[node];  // head hd drafted the children (depth hd + 1)
            lh = head_logits + ((int64_t)b * K + hd) * V;
            lse_h = head_lse[(int64_t)b * K + hd];
            double mass = 1.0, S = 1.0;
            for (int j = c0; j >= 0; j = next_sibling(t, j)) {
                const int x = tree_tok[(int64_t)b * N + j];
                if (x < 0 || x >= V) continue;  // not a token: never accepted, changes nothing
                const double px = (double)__expf(lt[x] * invT - lse_t);
                const double qx = (double)__expf(lh[x] * invT - lse_h);
                const double rx = fmax(0.0, px - c * qx);
                const double ratio = qx > 0.0 ? (rx / mass) * (S / qx) : INFINITY;
                const double u = (double)unit_f(u_words[(int64_t)b * N + j]);
                if (u < ratio) {
                    next = j;
                    break;
                }
                c += mass / S;
                S -= qx;
                if (next_sibling(t, j) >= 0) {  // another child may follow: the new residual's mass
                    const float cf = (float)c;
                    float acc = 0.0f;
                    for (int y = tid; y < V; y += WALK) {
                        const float p = __expf(lt[y] * invT - lse_t);
                        const float q = __expf(lh[y] * invT - lse_h);
                        acc += fmaxf(0.0f, p - cf * q);
                    }
                    mass = block_sum<WWAVES>((double)acc, shs);
                }
            }
        }
        if (next >= 0) {
            if (tid == 0) chosen[(int64_t)b * N + node] = tree_tok[(int64_t)b * N + next];
            node = next;
            continue;
        }
        // the step's last token: Gumbel-max over log R (a leaf: over log p)
        float bv = -INFINITY;
        int bi = INT_MAX;
        const float cf = (float)c;
        for (int y = tid; y < V; y += WALK) {
            float s;
            if (c0 < 0) {
                s = lt[y] * invT + gumbel_f(gw[y]);
            } else {
                const float p = __expf(lt[y] * invT - lse_t);
                const float q = __expf(lh[y] * invT - lse_h);
                const float r = p - cf * q;
                s = r > 0.0f ? __logf(r) + gumbel_f(gw[y]) : -INFINITY;
            }
            if (above(s, y, bv, bi)) {
                bv = s;
                bi = y;
            }
        }
        block_argmax<WWAVES>(bv, bi, shv, shi);
        if (tid == 0) chosen[(int64_t)b * N + node] = bi == INT_MAX ? -1 : bi;
        break;
    }
}

// ------------------------------------------------------- typical acceptance

// Block (request b, j-th node with children): log-sum-exp and entropy of the
// target's p at that node. H = lse - sum p z with z = l / T.
__global__ __launch_bounds__(BLOCK) void k_row_stats(DevTree t, int V, float invT, int P,
                                                     const float* __restrict__ target_logits,
                                                     float* __restrict__ lse_out, float* __restrict__ ent_out) {
    __shared__ float shm[NWAVE];
    __shared__ double shs[NWAVE];
    __shared__ int s_has[MD_WAVE], s_node;
    const int b = blockIdx.x / P, j = blockIdx.x - b * P;
    const int N = t.n;
    if (threadIdx.x < MD_WAVE) s_has[threadIdx.x] = 0;
    __syncthreads();
    if (threadIdx.x > 0 && threadIdx.x < N) s_has[t.parent[threadIdx.x]] = 1;
    __syncthreads();
    if (threadIdx.x < MD_WAVE) {
        // the j-th node with children, in node order
        uint64_t has = __ballot(s_has[threadIdx.x] != 0);
        for (int i = 0; i < j && has; ++i) has &= has - 1ull;
        if (threadIdx.x == 0) s_node = has ? __ffsll((long long)has) - 1 : -1;
    }
    __syncthreads();
    const int node = s_node;
    if (node < 0) return;  // uniform: fewer parents than blocks
    const float* lt = target_logits + ((int64_t)b * N + node) * V;
    float m = -INFINITY, s = 0.0f, wz = 0.0f;  // s = sum e^(z-m), wz = sum e^(z-m) z
    for (int y = threadIdx.x; y < V; y += BLOCK) {
        const float z = lt[y] * invT;
        if (z > m) {
            const float r = __expf(m - z);
            s = s * r + 1.0f;
            wz = wz * r + z;
            m = z;
        } else {
            const float e = __expf(z - m);
            s += e;
            wz += e * z;
        }
    }
    float bm = m;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) bm = fmaxf(bm, __shfl_xor(bm, o, MD_WAVE));
    if ((threadIdx.x & 63) == 0) shm[threadIdx.x >> 6] = bm;
    __syncthreads();
    float Mx = shm[0];
#pragma unroll
    for (int i = 1; i < NWAVE; ++i) Mx = fmaxf(Mx, shm[i]);
    const double f = s > 0.0f ? exp((double)m - (double)Mx) : 0.0;
    const double S = block_sum<NWAVE>((double)s * f, shs);
    const double W = block_sum<NWAVE>((double)wz * f, shs);
    if (threadIdx.x == 0) {
        const double lse = (double)Mx + log(S);
        lse_out[(int64_t)b * N + node] = (float)lse;
        ent_out[(int64_t)b * N + node] = (float)(lse - W / S);
    }
}

// One block per request: match bits (wave 0, one node per lane), the deepest
// accepted node, the tokens along its path, and the draw at that node.
__global__ __launch_bounds__(WALK) void k_typical(DevTree t, int V, float invT, float eps, float delta,
                                                  const float* __restrict__ target_logits,
                                                  const float* __restrict__ lse, const float* __restrict__ ent,
                                                  const int32_t* __restrict__ tree_tok,
                                                  const uint32_t* __restrict__ g_words,
                                                  int32_t* __restrict__ chosen) {
    __shared__ float shv[WWAVES];
    __shared__ int shi[WWAVES];
    __shared__ int s_a;
    const int b = blockIdx.x, N = t.n, tid = threadIdx.x;
    if (tid < MD_WAVE) {
        const int lane = tid;
        bool match = false;
        int tok = -1;
        if (lane < N) tok = tree_tok[(int64_t)b * N + lane];
        if (lane > 0 && lane < N && tok >= 0 && tok < V) {  // a value outside [0, V) never matches
            const int a = t.parent[lane];
            const int64_t ra = (int64_t)b * N + a;
            const double p = exp((double)(target_logits[ra * V + tok] * invT) - (double)lse[ra]);
            const double thr = fmin((double)eps, (double)delta * exp(-(double)ent[ra]));
            match = p > thr;
        }
        const uint64_t mset = __ballot(match);
        const uint64_t anc = lane < N ? t.anc[lane] : 0ull;
        const bool accepted = lane < N && ((anc & ~1ull) & ~mset) == 0ull;
        int key = accepted ? t.depth[lane] * 64 + (63 - lane) : -1;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) key = max(key, __shfl_xor(key, o, MD_WAVE));
        const int a = 63 - (key & 63);
        const uint64_t pa = __shfl(anc, a, MD_WAVE);
        // a node on the path (not the root) names its parent's emitted token
        const int child_on_path = [&] {
            int r = -1;
            for (int n = 1; n < N; ++n)
                if (((pa >> n) & 1ull) && t.parent[n] == lane) r = n;
            return r;
        }();
        const int ct = __shfl(tok, child_on_path < 0 ? 0 : child_on_path, MD_WAVE);  // the whole wave takes part
        if (lane < N) chosen[(int64_t)b * N + lane] = child_on_path >= 0 ? ct : -1;
        if (lane == 0) s_a = a;
    }
    __syncthreads();
    const int a = s_a;
    const float* lt = target_logits + ((int64_t)b * N + a) * V;
    const uint32_t* gw = g_words + (int64_t)b * V;
    float bv = -INFINITY;
    int bi = INT_MAX;
    for (int y = tid; y < V; y += WALK) {
        const float s = lt[y] * invT + gumbel_f(gw[y]);
        if (above(s, y, bv, bi)) {
            bv = s;
            bi = y;
        }
    }
    block_argmax<WWAVES>(bv, bi, shv, shi);
    if (tid == 0) chosen[(int64_t)b * N + a] = bi;
}

int count_parents(const DevTree& t) {
    int P = 0;
    for (int n = 0; n < t.n; ++n) {
        bool has = false;
        for (int c = n + 1; c < t.n; ++c) has |= t.parent[c] == n;
        P += has;
    }
    return P;
}

}  // namespace

size_t draft_sample_ws_bytes(int M, int K, int V, int kmax) {
    const size_t rows = (size_t)M * K, ch = (size_t)draft_chunks(M * K, V);
    return 2 * align256(rows * ch * kmax * 4) + align256(rows * ch * 4) + align256(rows * kmax * 4);
}

hipError_t draft_sample_launch(int M, int K, int V, const int* kk, int kmax, float T, const float* logits,
                               const uint32_t* words, int32_t* tok, float* lse, void* ws, hipStream_t s) {
    const int rows = M * K, ch = draft_chunks(rows, V);
    char* w = reinterpret_cast<char*>(ws);
    float* pv = reinterpret_cast<float*>(w);
    w += align256((size_t)rows * ch * kmax * 4);
    int* pi = reinterpret_cast<int*>(w);
    w += align256((size_t)rows * ch * kmax * 4);
    float* pl = reinterpret_cast<float*>(w);
    w += align256((size_t)rows * ch * 4);
    float* score = reinterpret_cast<float*>(w);
    KS ks;
    for (int i = 0; i < 8; ++i) ks.v[i] = i < K ? kk[i] : 1;
    hipLaunchKernelGGL(k_draft_part, dim3((unsigned)(rows * ch)), dim3(BLOCK), 0, s, logits, words, M, K, V, 1.0f / T,
                       ch, ks, kmax, pv, pi, pl);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_lse_merge, dim3((rows + 255) / 256), dim3(256), 0, s, pl, rows, ch, lse);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return topk_merge_launch(pv, pi, M, K, ch, kk, kmax, tok, score, s);
}

size_t verify_sampled_ws_bytes(int B, int N) { return align256((size_t)B * N * 4); }

hipError_t verify_sampled_launch(const DevTree& t, int dt, int B, int K, int V, int Hkv, int hd, int Lcap, float T,
                                 const float* target_logits, const float* head_logits, const float* head_lse,
                                 const int32_t* tree_tok, const uint32_t* u_words, const uint32_t* g_words,
                                 void* Kc, void* Vc, int32_t* lens, int32_t* accept_len, int32_t* path,
                                 int32_t* next_tok, int32_t* compact_src, void* ws, hipStream_t s) {
    int32_t* chosen = reinterpret_cast<int32_t*>(ws);
    hipLaunchKernelGGL(k_walk_sampled, dim3(B), dim3(WALK), 0, s, t, K, V, 1.0f / T, target_logits, head_logits,
                       head_lse, tree_tok, u_words, g_words, chosen);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return accept_tokens_launch(t, dt, B, K, Hkv, hd, Lcap, chosen, tree_tok, Kc, Vc, lens, accept_len, path,
                                next_tok, compact_src, s);
}

size_t accept_typical_ws_bytes(int B, int N) { return 3 * align256((size_t)B * N * 4); }

hipError_t accept_typical_launch(const DevTree& t, int dt, int B, int K, int V, int Hkv, int hd, int Lcap, float T,
                                 float eps, float delta, const float* target_logits, const int32_t* tree_tok,
                                 const uint32_t* g_words, void* Kc, void* Vc, int32_t* lens, int32_t* accept_len,
                                 int32_t* path, int32_t* next_tok, int32_t* compact_src, void* ws, hipStream_t s) {
    char* w = reinterpret_cast<char*>(ws);
    int32_t* chosen = reinterpret_cast<int32_t*>(w);
    w += align256((size_t)B * t.n * 4);
    float* lse = reinterpret_cast<float*>(w);
    w += align256((size_t)B * t.n * 4);
    float* ent = reinterpret_cast<float*>(w);
    const int P = count_parents(t);
    const float invT = 1.0f / T;
    if (P > 0) {
        hipLaunchKernelGGL(k_row_stats, dim3((unsigned)(B * P)), dim3(BLOCK), 0, s, t, V, invT, P, target_logits, lse,
                           ent);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_typical, dim3(B), dim3(WALK), 0, s, t, V, invT, eps, delta, target_logits, lse, ent,
                       tree_tok, g_words, chosen);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return accept_tokens_launch(t, dt, B, K, Hkv, hd, Lcap, chosen, tree_tok, Kc, Vc, lens, accept_len, path,
                                next_tok, compact_src, s);
}
