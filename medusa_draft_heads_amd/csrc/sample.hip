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
#include "md_wave.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

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
    bm = md_wave::wave_max(bm);
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
    md_wave::wave_argmax(v, i);
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
    // v[i] with no memory access: a kernel argument indexed by a runtime
    // value is read with a vector load, and waiting for that load also waits
    // for every store the wave still has in flight (stores share the counter).
    // Each v[j] is read with a constant index (a scalar load) and made opaque
    // to the compiler, which would otherwise turn the selects back into an
    // indexed load.
    __device__ __forceinline__ int at(int i) const {
        int r = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            int x = v[j];
            asm volatile("" : "+s"(x));
            r = i == j ? x : r;
        }
        return r;
    }
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
    const int k = ks.at(h);
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
    auto take = [&](int y, float l, uint32_t word) {
        const float z = l * invT;
        lse_add(lm, ls, z);
        const float s = z + gumbel_f(word);
        if (!above(s, y, v[KM - 1], ix[KM - 1])) return;
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
    };
    // 8 logits and words loaded per thread before they are taken, in the same
    // order as one at a time (past the chunk's end the loads repeat its last
    // element and are not taken)
    for (int y0 = a + tid; y0 < e; y0 += 8 * BLOCK) {
        float lv[8];
        uint32_t wv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int y = min(y0 + u * BLOCK, e - 1);
            lv[u] = lg[y];
            wv[u] = wd[y];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (y0 + u * BLOCK < e) take(y0 + u * BLOCK, lv[u], wv[u]);
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

// One wave per row-head: log-sum-exp of the chunks' log-sum-exps.
__global__ __launch_bounds__(MD_WAVE) void k_lse_merge(const float* __restrict__ part_lse, int chunks,
                                                       float* __restrict__ lse) {
    const int r = blockIdx.x, lane = threadIdx.x;
    const float* pl = part_lse + (int64_t)r * chunks;
    float m = -INFINITY;
    for (int c = lane; c < chunks; c += MD_WAVE) m = fmaxf(m, pl[c]);
    m = md_wave::wave_max(m);
    double S = 0.0;
    for (int c = lane; c < chunks; c += MD_WAVE)
        if (pl[c] > -INFINITY) S += exp((double)pl[c] - (double)m);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) S += __shfl_xor(S, o, MD_WAVE);
    if (lane == 0) lse[r] = (float)((double)m + log(S));
}

int draft_chunks(int rows, int V) {
    int c = (kDraftBlocks + rows - 1) / rows;
    const int max_c = (V + BLOCK - 1) / BLOCK;  // at least a thread's worth each
    if (c > max_c) c = max_c;
    return c < 1 ? 1 : c;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ------------------------------------------------------------- the walk

// The nodes with children, in node order (passed by value).
struct Parents {
    int n;
    int8_t node[64];
};

Parents parents_of(const DevTree& t) {
    Parents p;
    p.n = 0;
    for (int n = 0; n < t.n; ++n) {
        bool has = false;
        for (int c = n + 1; c < t.n; ++c) has |= t.parent[c] == n;
        if (has) p.node[p.n++] = (int8_t)n;
    }
    return p;
}

// What the step's last draw samples from: the target at `node`, and with
// head >= 0 the residual max(0, p - c q) against that head's q.
struct DrawSpec {
    int node;
    int head;
    float c;
    float lse_t;
    float lse_h;
};

constexpr int kStatBlocks = 2048;  // row statistics: blocks over all rows
constexpr int kDrawBlocks = 1024;  // final draws: blocks over all requests

int split_chunks(int rows, int V, int target_blocks) {
    int c = (target_blocks + rows - 1) / rows;
    const int max_c = (V + 16 * BLOCK - 1) / (16 * BLOCK);  // at least 16 elements a thread
    if (c > max_c) c = max_c;
    return c < 1 ? 1 : c;
}

// Calls f(y, x) for every element y of row x[] in [a, e): 16-byte loads,
// eight in flight per thread, when rows are 16-byte aligned (V % 4 == 0);
// each thread visits its elements in increasing order either way (past the
// range's end the loads repeat its last 16 bytes and are not visited).
template <int NT, typename F>
__device__ __forceinline__ void sweep(const float* __restrict__ x, int V, int a, int e, F&& f) {
    const int tid = threadIdx.x;
    if ((V & 3) == 0) {
        const f32x4* x4 = reinterpret_cast<const f32x4*>(x);
        const int a4 = (a + 3) >> 2, e4 = e >> 2;  // chunks split on multiples of 4 below
        for (int j = a4 + tid; j < e4; j += 8 * NT) {
            f32x4 u[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) u[q] = x4[min(j + q * NT, e4 - 1)];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int k = j + q * NT;
                if (k < e4) {
                    f(4 * k, u[q].x); f(4 * k + 1, u[q].y); f(4 * k + 2, u[q].z); f(4 * k + 3, u[q].w);
                }
            }
        }
    } else {
        for (int y = a + tid; y < e; y += NT) f(y, x[y]);
    }
}

// chunk ch of nc over [0, V): bounds on multiples of 4 so the 16-byte sweep covers it exactly
__device__ __forceinline__ void chunk_range(int V, int ch, int nc, int& a, int& e) {
    const int V4 = (V + 3) >> 2;
    a = (int)((int64_t)V4 * ch / nc) * 4;
    e = min(V, (int)((int64_t)V4 * (ch + 1) / nc) * 4);
}

// Block (row r = (request b, j-th parent), chunk ch): the chunk's
// (largest z, sum e^(z - m), sum e^(z - m) z) with z = l / T.
__global__ __launch_bounds__(BLOCK) void k_row_stats_part(Parents pl, int N, int V, float invT, int chunks,
                                                          const float* __restrict__ target_logits,
                                                          float* __restrict__ part) {
    __shared__ float shm[NWAVE];
    __shared__ double shs[NWAVE];
    const int r = blockIdx.x / chunks, ch = blockIdx.x - r * chunks;
    const int b = r / pl.n, node = pl.node[r - b * pl.n];
    const float* lt = target_logits + ((int64_t)b * N + node) * V;
    int a, e;
    chunk_range(V, ch, chunks, a, e);
    float m = -INFINITY, s = 0.0f, wz = 0.0f;
    sweep<BLOCK>(lt, V, a, e, [&](int, float l) {
        const float z = l * invT;
        if (z > m) {
            const float q = __expf(m - z);
            s = s * q + 1.0f;
            wz = wz * q + z;
            m = z;
        } else {
            const float q = __expf(z - m);
            s += q;
            wz += q * z;
        }
    });
    float bm = m;
    bm = md_wave::wave_max(bm);
    if ((threadIdx.x & 63) == 0) shm[threadIdx.x >> 6] = bm;
    __syncthreads();
    float M = shm[0];
#pragma unroll
    for (int i = 1; i < NWAVE; ++i) M = fmaxf(M, shm[i]);
    const double f = s > 0.0f ? exp((double)m - (double)M) : 0.0;
    const double S = block_sum<NWAVE>((double)s * f, shs);
    const double W = block_sum<NWAVE>((double)wz * f, shs);
    if (threadIdx.x == 0) {
        float* o = part + ((int64_t)r * chunks + ch) * 3;
        o[0] = M;
        o[1] = (float)S;
        o[2] = (float)W;
    }
}

// One wave per row: combine the chunks; lse = M + log S, entropy = lse - W / S.
__global__ __launch_bounds__(MD_WAVE) void k_row_stats_merge(Parents pl, int N, int chunks,
                                                             const float* __restrict__ part,
                                                             float* __restrict__ lse_out,
                                                             float* __restrict__ ent_out) {
    const int r = blockIdx.x, lane = threadIdx.x;
    const int b = r / pl.n, node = pl.node[r - b * pl.n];
    const float* pr = part + (int64_t)r * chunks * 3;
    float M = -INFINITY;
    for (int c = lane; c < chunks; c += MD_WAVE) M = fmaxf(M, pr[3 * c]);
    M = md_wave::wave_max(M);
    double S = 0.0, W = 0.0;
    for (int c = lane; c < chunks; c += MD_WAVE) {
        if (pr[3 * c + 1] > 0.0f) {
            const double f = exp((double)pr[3 * c] - (double)M);
            S += (double)pr[3 * c + 1] * f;
            W += (double)pr[3 * c + 2] * f;
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        S += __shfl_xor(S, o, MD_WAVE);
        W += __shfl_xor(W, o, MD_WAVE);
    }
    if (lane == 0) {
        const double lse = (double)M + log(S);
        lse_out[(int64_t)b * N + node] = (float)lse;
        if (ent_out) ent_out[(int64_t)b * N + node] = (float)(lse - W / S);
    }
}

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
// scalars; the residual masses are block reductions over the vocabulary.
// The walk ends by describing the last draw (spec), made by k_draw_*.
__global__ __launch_bounds__(WALK) void k_walk_sampled(DevTree t, int K, int V, float invT,
                                                       const float* __restrict__ target_logits,
                                                       const float* __restrict__ head_logits,
                                                       const float* __restrict__ head_lse,
                                                       const float* __restrict__ lse_rows,
                                                       const int32_t* __restrict__ tree_tok,
                                                       const uint32_t* __restrict__ u_words,
                                                       int32_t* __restrict__ chosen, DrawSpec* __restrict__ spec) {
    __shared__ double shs[WWAVES];
    const int b = blockIdx.x, N = t.n, tid = threadIdx.x;
    if (tid < N) chosen[(int64_t)b * N + tid] = -1;
    __syncthreads();  // thread 0 may later write any node's entry
    int node = 0;
    while (true) {
        const int c0 = first_child(t, node);
        if (c0 < 0) {  // a leaf: the last token is drawn from p
            if (tid == 0) spec[b] = DrawSpec{node, -1, 0.0f, 0.0f, 0.0f};
            return;
        }
        const float* lt = target_logits + ((int64_t)b * N + node) * V;
        const float lse_t = lse_rows[(int64_t)b * N + node];
        const int hd = t.depth[node];  // head hd drafted the children (depth hd + 1)
        const float* lh = head_logits + ((int64_t)b * K + hd) * V;
        const float lse_h = head_lse[(int64_t)b * K + hd];
        double c = 0.0, mass = 1.0, S = 1.0;  // residual R(y) = max(0, p(y) - c q(y)), mass M, q-mass S
        int next = -1;
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
                if ((V & 3) == 0) {
                    const f32x4* lt4 = reinterpret_cast<const f32x4*>(lt);
                    const f32x4* lh4 = reinterpret_cast<const f32x4*>(lh);
                    const int V4 = V >> 2;
                    int i = tid;
                    for (; i + WALK < V4; i += 2 * WALK) {
                        const f32x4 ta = lt4[i], ha = lh4[i], tb = lt4[i + WALK], hb = lh4[i + WALK];
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            acc += fmaxf(0.0f, __expf(ta[q] * invT - lse_t) - cf * __expf(ha[q] * invT - lse_h));
                            acc += fmaxf(0.0f, __expf(tb[q] * invT - lse_t) - cf * __expf(hb[q] * invT - lse_h));
                        }
                    }
                    if (i < V4) {
                        const f32x4 ta = lt4[i], ha = lh4[i];
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            acc += fmaxf(0.0f, __expf(ta[q] * invT - lse_t) - cf * __expf(ha[q] * invT - lse_h));
                    }
                } else {
                    for (int y = tid; y < V; y += WALK)
                        acc += fmaxf(0.0f, __expf(lt[y] * invT - lse_t) - cf * __expf(lh[y] * invT - lse_h));
                }
                mass = block_sum<WWAVES>((double)acc, shs);
            }
        }
        if (next >= 0) {
            if (tid == 0) chosen[(int64_t)b * N + node] = tree_tok[(int64_t)b * N + next];
            node = next;
            continue;
        }
        if (tid == 0) spec[b] = DrawSpec{node, hd, (float)c, lse_t, lse_h};  // every child rejected
        return;
    }
}

// The last draws: Gumbel-max over log R (or log p), split over the
// vocabulary; block (request b, chunk ch) leaves its best (value, index).
__global__ __launch_bounds__(BLOCK) void k_draw_part(int N, int K, int V, float invT, int chunks,
                                                     const DrawSpec* __restrict__ spec,
                                                     const float* __restrict__ target_logits,
                                                     const float* __restrict__ head_logits,
                                                     const uint32_t* __restrict__ g_words,
                                                     float* __restrict__ pv, int* __restrict__ pi) {
    __shared__ float shv[NWAVE];
    __shared__ int shi[NWAVE];
    const int b = blockIdx.x / chunks, ch = blockIdx.x - b * chunks;
    const DrawSpec sp = spec[b];
    const float* lt = target_logits + ((int64_t)b * N + sp.node) * V;
    const float* lh = sp.head >= 0 ? head_logits + ((int64_t)b * K + sp.head) * V : nullptr;
    const uint32_t* gw = g_words + (int64_t)b * V;
    int a, e;
    chunk_range(V, ch, chunks, a, e);
    float bv = -INFINITY;
    int bi = INT_MAX;
    if (sp.head < 0) {
        sweep<BLOCK>(lt, V, a, e, [&](int y, float l) {
            const float s = l * invT + gumbel_f(gw[y]);
            if (above(s, y, bv, bi)) {
                bv = s;
                bi = y;
            }
        });
    } else {
        sweep<BLOCK>(lt, V, a, e, [&](int y, float l) {
            const float r = __expf(l * invT - sp.lse_t) - sp.c * __expf(lh[y] * invT - sp.lse_h);
            if (r > 0.0f) {
                const float s = __logf(r) + gumbel_f(gw[y]);
                if (above(s, y, bv, bi)) {
                    bv = s;
                    bi = y;
                }
            }
        });
    }
    block_argmax<NWAVE>(bv, bi, shv, shi);
    if (threadIdx.x == 0) {
        pv[blockIdx.x] = bv;
        pi[blockIdx.x] = bi;
    }
}

// One wave per request: the best of the chunks is the token after spec.node.
__global__ __launch_bounds__(MD_WAVE) void k_draw_merge(int N, int chunks, const DrawSpec* __restrict__ spec,
                                                        const float* __restrict__ pv, const int* __restrict__ pi,
                                                        int32_t* __restrict__ chosen) {
    const int b = blockIdx.x, lane = threadIdx.x;
    float bv = -INFINITY;
    int bi = INT_MAX;
    for (int c = lane; c < chunks; c += MD_WAVE) {
        const float v = pv[(int64_t)b * chunks + c];
        const int i = pi[(int64_t)b * chunks + c];
        if (above(v, i, bv, bi)) {
            bv = v;
            bi = i;
        }
    }
    md_wave::wave_argmax(bv, bi);
    if (lane == 0) chosen[(int64_t)b * N + spec[b].node] = bi == INT_MAX ? -1 : bi;
}

// ------------------------------------------------------- typical acceptance

// One wave per request: match bits (one node per lane), the deepest accepted
// node, the tokens along its path; the last draw is at that node's p.
__global__ __launch_bounds__(MD_WAVE) void k_typical(DevTree t, int V, float invT, float eps, float delta,
                                                     const float* __restrict__ target_logits,
                                                     const float* __restrict__ lse, const float* __restrict__ ent,
                                                     const int32_t* __restrict__ tree_tok,
                                                     int32_t* __restrict__ chosen, DrawSpec* __restrict__ spec) {
    const int b = blockIdx.x, N = t.n, lane = threadIdx.x;
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
    key = md_wave::wave_max(key);
    const int a = 63 - (key & 63);
    const uint64_t pa = __shfl(anc, a, MD_WAVE);
    // a node on the path (not the root) names its parent's emitted token
    int child_on_path = -1;
    for (int n = 1; n < N; ++n)
        if (((pa >> n) & 1ull) && t.parent[n] == lane) child_on_path = n;
    const int ct = __shfl(tok, child_on_path < 0 ? 0 : child_on_path, MD_WAVE);  // the whole wave takes part
    if (lane < N) chosen[(int64_t)b * N + lane] = child_on_path >= 0 ? ct : -1;
    if (lane == 0) spec[b] = DrawSpec{a, -1, 0.0f, 0.0f, 0.0f};
}

// Workspace of both verifiers: chosen [B][N], lse and entropy [B][N], the
// row-statistics partials, the draw specs and the draw partials.
struct VerifyWs {
    int32_t* chosen;
    float* lse;
    float* ent;
    float* stat_part;
    DrawSpec* spec;
    float* draw_v;
    int* draw_i;
};

VerifyWs verify_ws_layout(void* base, int B, int N, size_t* total) {
    char* w = reinterpret_cast<char*>(base);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* p = w ? w + off : nullptr;
        off += align256(bytes);
        return p;
    };
    VerifyWs L;
    L.chosen = reinterpret_cast<int32_t*>(take((size_t)B * N * 4));
    L.lse = reinterpret_cast<float*>(take((size_t)B * N * 4));
    L.ent = reinterpret_cast<float*>(take((size_t)B * N * 4));
    // rows x chunks <= kStatBlocks + rows whatever V is (chunks = ceil(kStatBlocks / rows) at most)
    L.stat_part = reinterpret_cast<float*>(take(((size_t)kStatBlocks + (size_t)B * N) * 3 * 4));
    L.spec = reinterpret_cast<DrawSpec*>(take((size_t)B * sizeof(DrawSpec)));
    L.draw_v = reinterpret_cast<float*>(take(((size_t)kDrawBlocks + B) * 4));
    L.draw_i = reinterpret_cast<int*>(take(((size_t)kDrawBlocks + B) * 4));
    if (total) *total = off;
    return L;
}

hipError_t row_stats_launch(const Parents& pl, int B, int N, int V, float invT, const float* target_logits,
                            const VerifyWs& L, bool entropy, hipStream_t s) {
    if (pl.n == 0) return hipSuccess;
    const int rows = B * pl.n, ch = split_chunks(rows, V, kStatBlocks);
    hipLaunchKernelGGL(k_row_stats_part, dim3((unsigned)(rows * ch)), dim3(BLOCK), 0, s, pl, N, V, invT, ch,
                       target_logits, L.stat_part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_row_stats_merge, dim3((unsigned)rows), dim3(MD_WAVE), 0, s, pl, N, ch, L.stat_part, L.lse,
                       entropy ? L.ent : nullptr);
    return hipGetLastError();
}

hipError_t draw_launch(int B, int N, int K, int V, float invT, const float* target_logits, const float* head_logits,
                       const uint32_t* g_words, const VerifyWs& L, hipStream_t s) {
    const int ch = split_chunks(B, V, kDrawBlocks);
    hipLaunchKernelGGL(k_draw_part, dim3((unsigned)(B * ch)), dim3(BLOCK), 0, s, N, K, V, invT, ch, L.spec,
                       target_logits, head_logits, g_words, L.draw_v, L.draw_i);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_draw_merge, dim3((unsigned)B), dim3(MD_WAVE), 0, s, N, ch, L.spec, L.draw_v, L.draw_i,
                       L.chosen);
    return hipGetLastError();
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
    hipLaunchKernelGGL(k_lse_merge, dim3(rows), dim3(MD_WAVE), 0, s, pl, ch, lse);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return topk_merge_launch(pv, pi, M, K, ch, kk, kmax, tok, score, s);
}

size_t verify_sampled_ws_bytes(int B, int N) {
    size_t total = 0;
    verify_ws_layout(nullptr, B, N, &total);
    return total;
}

hipError_t verify_sampled_launch(const DevTree& t, int dt, int B, int K, int V, int Hkv, int hd, int Lcap, float T,
                                 const float* target_logits, const float* head_logits, const float* head_lse,
                                 const int32_t* tree_tok, const uint32_t* u_words, const uint32_t* g_words,
                                 void* Kc, void* Vc, int32_t* lens, int32_t* accept_len, int32_t* path,
                                 int32_t* next_tok, int32_t* compact_src, void* ws, hipStream_t s) {
    const VerifyWs L = verify_ws_layout(ws, B, t.n, nullptr);
    const float invT = 1.0f / T;
    const Parents pl = parents_of(t);
    hipError_t e = row_stats_launch(pl, B, t.n, V, invT, target_logits, L, false, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_walk_sampled, dim3(B), dim3(WALK), 0, s, t, K, V, invT, target_logits, head_logits,
                       head_lse, L.lse, tree_tok, u_words, L.chosen, L.spec);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = draw_launch(B, t.n, K, V, invT, target_logits, head_logits, g_words, L, s);
    if (e != hipSuccess) return e;
    return accept_tokens_launch(t, dt, B, K, Hkv, hd, Lcap, L.chosen, tree_tok, Kc, Vc, lens, accept_len, path,
                                next_tok, compact_src, s);
}

size_t accept_typical_ws_bytes(int B, int N) { return verify_sampled_ws_bytes(B, N); }

hipError_t accept_typical_launch(const DevTree& t, int dt, int B, int K, int V, int Hkv, int hd, int Lcap, float T,
                                 float eps, float delta, const float* target_logits, const int32_t* tree_tok,
                                 const uint32_t* g_words, void* Kc, void* Vc, int32_t* lens, int32_t* accept_len,
                                 int32_t* path, int32_t* next_tok, int32_t* compact_src, void* ws, hipStream_t s) {
    const VerifyWs L = verify_ws_layout(ws, B, t.n, nullptr);
    const float invT = 1.0f / T;
    const Parents pl = parents_of(t);
    hipError_t e = row_stats_launch(pl, B, t.n, V, invT, target_logits, L, true, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_typical, dim3(B), dim3(MD_WAVE), 0, s, t, V, invT, eps, delta, target_logits, L.lse, L.ent,
                       tree_tok, L.chosen, L.spec);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = draw_launch(B, t.n, K, V, invT, target_logits, nullptr, g_words, L, s);
    if (e != hipSuccess) return e;
    return accept_tokens_launch(t, dt, B, K, Hkv, hd, Lcap, L.chosen, tree_tok, Kc, Vc, lens, accept_len, path,
                                next_tok, compact_src, s);
}
