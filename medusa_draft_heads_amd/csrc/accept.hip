// Greedy verification, the longest accepted branch, and cache compaction.
//
// "Medusa heads versus separate draft model", section "Trees": if a branch of
// the tree matches the target, the step advances along it; section
// "Acceptance": the step yields the target's own token plus the accepted
// drafts. Greedy matching: a draft node matches when its token is the
// target's argmax at its parent; a node is accepted when its whole root path
// matches. Siblings carry distinct tokens, so the accepted nodes form one
// chain; its deepest node ends the step.
//
// k_argmax_part: the target's choice per (request, node) row, split over
// chunks of the vocabulary so the 4-byte logits stream at full bandwidth
// (first maximal index wins). k_accept: one block per request. Wave 0 holds
// one node per lane: match bits come from one ballot, "accepted" is
// (ancestor set minus root) within the match set, and the deepest accepted
// node is a wave max over (depth, -index). The branch's cache entries then
// move next to the prefix: every source slot is read into LDS before any
// destination is written, because a source can be a later destination.
#include <math.h>

#include "md_internal.h"
#include "md_wave.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BLOCK = 256;
constexpr int NWAVE = BLOCK / MD_WAVE;
constexpr int kTargetBlocks = 1024;
constexpr int kCompactLds = 32 * 1024;  // bytes of LDS staging for the compaction

__device__ __forceinline__ bool beats(float v, int i, float w, int j) { return v > w || (v == w && i < j); }

__device__ __forceinline__ void wave_argmax(float& v, int& i) {
    md_wave::wave_argmax(v, i);
}

__global__ __launch_bounds__(BLOCK) void k_argmax_part(const float* __restrict__ logits, int V, int chunks,
                                                       float* __restrict__ part_v, int* __restrict__ part_i) {
    __shared__ float sv[NWAVE];
    __shared__ int si[NWAVE];
    const int64_t row = blockIdx.x / chunks;
    const int ch = blockIdx.x - (int)(row * chunks);
    const float* x = logits + row * V;
    float bv = -INFINITY;
    int bi = INT_MAX;
    if ((V & 3) == 0) {
        const int V4 = V >> 2;
        const int a = (int)((int64_t)V4 * ch / chunks), e = (int)((int64_t)V4 * (ch + 1) / chunks);
        const f32x4* x4 = reinterpret_cast<const f32x4*>(x);
        auto take = [&](const f32x4& v, int j) {
            const int i0 = 4 * j;
            if (beats(v.x, i0, bv, bi)) { bv = v.x; bi = i0; }
            if (beats(v.y, i0 + 1, bv, bi)) { bv = v.y; bi = i0 + 1; }
            if (beats(v.z, i0 + 2, bv, bi)) { bv = v.z; bi = i0 + 2; }
            if (beats(v.w, i0 + 3, bv, bi)) { bv = v.w; bi = i0 + 3; }
        };
        // 8 loads in flight per thread before any compare ("beats" is a total
        // order, so the order the entries are visited in does not matter);
        // past the chunk's end a load repeats its last chunk of 4 (in bounds)
        // and is not compared
        for (int j = a + (int)threadIdx.x; j < e; j += 8 * BLOCK) {
            f32x4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(x4 + min(j + u * BLOCK, e - 1));
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (j + u * BLOCK < e) take(v[u], j + u * BLOCK);
        }
    } else {
        const int a = (int)((int64_t)V * ch / chunks), e = (int)((int64_t)V * (ch + 1) / chunks);
        for (int j = a + threadIdx.x; j < e; j += BLOCK) {
            const float v = x[j];
            if (beats(v, j, bv, bi)) { bv = v; bi = j; }
        }
    }
    wave_argmax(bv, bi);
    const int lane = threadIdx.x & (MD_WAVE - 1), w = threadIdx.x >> 6;
    if (lane == 0) {
        sv[w] = bv;
        si[w] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        bv = sv[0];
        bi = si[0];
        for (int k = 1; k < NWAVE; ++k)
            if (beats(sv[k], si[k], bv, bi)) {
                bv = sv[k];
                bi = si[k];
            }
        part_v[blockIdx.x] = bv;
        part_i[blockIdx.x] = bi;
    }
}

// The target's choice per node comes from the argmax parts (chunks per row),
// or ready-made from target_tok [B][N] when that is given.
template <typename T>
__global__ __launch_bounds__(BLOCK) void k_accept(DevTree t, int K, int Hkv, int hd, int Lcap, int chunks,
                                                  const float* __restrict__ part_v, const int* __restrict__ part_i,
                                                  const int32_t* __restrict__ target_tok,
                                                  const int32_t* __restrict__ tree_tok, T* __restrict__ Kc,
                                                  T* __restrict__ Vc, int32_t* __restrict__ lens,
                                                  int32_t* __restrict__ accept_len, int32_t* __restrict__ path,
                                                  int32_t* __restrict__ next_tok, int32_t* __restrict__ compact_src) {
    __shared__ int s_path[64];
    __shared__ int s_A, s_L, s_ok;
    extern __shared__ __align__(16) unsigned char s_buf[];  // [2][K+1][hd] elements of T
    const int b = blockIdx.x;
    const int N = t.n;
    const int tid = threadIdx.x, lane = tid & (MD_WAVE - 1);
    if (tid < MD_WAVE) {
        const int L = lens[b];
        const bool ok = L >= 0 && (int64_t)L + N <= Lcap;
        // the target's choice at this lane's node
        float bv = -INFINITY;
        int bi = INT_MAX;
        if (target_tok) {
            if (lane < N) bi = target_tok[(int64_t)b * N + lane];
        } else if (lane < N) {
            const int64_t r = ((int64_t)b * N + lane) * chunks;
            for (int c0 = 0; c0 < chunks; c0 += 8) {
                float v[8];
                int ix[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    v[u] = c0 + u < chunks ? part_v[r + c0 + u] : -INFINITY;
                    ix[u] = c0 + u < chunks ? part_i[r + c0 + u] : INT_MAX;
                }
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (beats(v[u], ix[u], bv, bi)) {
                        bv = v[u];
                        bi = ix[u];
                    }
            }
        }
        const int tstar = bi;
        const int par = lane < N ? t.parent[lane] : -1;
        const int tstar_par = __shfl(tstar, par < 0 ? 0 : par, MD_WAVE);
        const int tok = lane < N ? tree_tok[(int64_t)b * N + lane] : -1;
        const bool match = lane > 0 && lane < N && tok == tstar_par;
        const uint64_t mset = __ballot(match);
        const uint64_t anc = lane < N ? t.anc[lane] : 0ull;
        const bool accepted = lane < N && ((anc & ~1ull) & ~mset) == 0ull;
        const int dep = lane < N ? t.depth[lane] : 0;
        // deepest accepted node, lowest index among equals: maximise depth*64 + (63 - lane)
        int key = accepted ? dep * 64 + (63 - lane) : -1;
        key = md_wave::wave_max(key);
        const int a = 63 - (key & 63);
        const int da = key >> 6;
        const uint64_t pa = __shfl(anc, a, MD_WAVE);  // a's root path as a node set
        const int nt = __shfl(tstar, a, MD_WAVE);
        // path[j] = the j-th member of pa in index order (breadth-first
        // numbering puts a node's ancestors in depth order); pa has da + 1 members
        const int A = ok ? da + 1 : 0;
        if (lane <= K) {
            int node = -1;
            if (lane < A) {
                uint64_t x = pa;
                for (int i = 0; i < lane; ++i) x &= x - 1ull;
                node = __ffsll((long long)x) - 1;
            }
            s_path[lane] = node;
            path[(int64_t)b * (K + 1) + lane] = node;
            compact_src[(int64_t)b * (K + 1) + lane] = node >= 0 ? L + node : -1;
        }
        if (lane == 0) {
            s_ok = ok;
            s_L = L;
            s_A = A;
            accept_len[b] = A;
            next_tok[b] = ok ? nt : -1;
        }
    }
    __syncthreads();
    if (!s_ok) return;
    const int A = s_A, L = s_L;
    const int row_bytes = hd * (int)sizeof(T);
    if ((row_bytes & 15) == 0) {
        // 16-byte chunks: a slot row is row_bytes / 16 chunks
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        u32x4* buf = reinterpret_cast<u32x4*>(s_buf);
        const int cpr = row_bytes >> 4;
        const int per = A * cpr;  // chunks per kv head and per tensor
        const int gstep = max(1, kCompactLds / (2 * (K + 1) * row_bytes));
        for (int g0 = 0; g0 < Hkv; g0 += gstep) {
            const int ng = min(gstep, Hkv - g0);
            const int tot = ng * 2 * per;
            for (int i = tid; i < tot; i += BLOCK) {
                const int gi = i / (2 * per), rem = i - gi * 2 * per;
                const int which = rem / per, r = rem - which * per;
                const int jj = r / cpr, c = r - jj * cpr;
                const int64_t base = ((int64_t)b * Hkv + g0 + gi) * Lcap;
                const T* src = which ? Vc : Kc;
                buf[i] = reinterpret_cast<const u32x4*>(src + (base + L + s_path[jj]) * hd)[c];
            }
            __syncthreads();
            for (int i = tid; i < tot; i += BLOCK) {
                const int gi = i / (2 * per), rem = i - gi * 2 * per;
                const int which = rem / per, r = rem - which * per;
                const int jj = r / cpr, c = r - jj * cpr;
                const int64_t base = ((int64_t)b * Hkv + g0 + gi) * Lcap;
                T* dst = which ? Vc : Kc;
                reinterpret_cast<u32x4*>(dst + (base + L + jj) * hd)[c] = buf[i];
            }
            __syncthreads();
        }
    } else {
        T* buf = reinterpret_cast<T*>(s_buf);
        const int per = A * hd;  // elements per kv head and per tensor
        const int gstep = max(1, kCompactLds / (2 * (K + 1) * row_bytes));
        for (int g0 = 0; g0 < Hkv; g0 += gstep) {
            const int ng = min(gstep, Hkv - g0);
            const int tot = ng * 2 * per;
            for (int i = tid; i < tot; i += BLOCK) {
                const int gi = i / (2 * per), rem = i - gi * 2 * per;
                const int which = rem / per, r = rem - which * per;
                const int jj = r / hd, c = r - jj * hd;
                const int64_t base = ((int64_t)b * Hkv + g0 + gi) * Lcap;
                const T* src = which ? Vc : Kc;
                buf[i] = src[(base + L + s_path[jj]) * hd + c];
            }
            __syncthreads();
            for (int i = tid; i < tot; i += BLOCK) {
                const int gi = i / (2 * per), rem = i - gi * 2 * per;
                const int which = rem / per, r = rem - which * per;
                const int jj = r / hd, c = r - jj * hd;
                const int64_t base = ((int64_t)b * Hkv + g0 + gi) * Lcap;
                T* dst = which ? Vc : Kc;
                dst[(base + L + jj) * hd + c] = buf[i];
            }
            __syncthreads();
        }
    }
    if (tid == 0) lens[b] = L + A;
}

int pick_chunks(int rows, int V) {
    int c = (kTargetBlocks + rows - 1) / rows;
    const int max_c = (V + 4 * BLOCK - 1) / (4 * BLOCK);  // at least one float4 per thread
    if (c > max_c) c = max_c;
    return c < 1 ? 1 : c;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t accept_ws_bytes(int B, int N, int V) {
    const size_t parts = (size_t)B * N * pick_chunks(B * N, V);
    return 2 * align256(parts * 4);
}

hipError_t accept_launch(const DevTree& t, int dt, int B, int K, int V, int Hkv, int hd, int Lcap,
                         const float* logits, const int32_t* tree_tok, void* Kc, void* Vc, int32_t* lens,
                         int32_t* accept_len, int32_t* path, int32_t* next_tok, int32_t* compact_src, void* ws,
                         hipStream_t s) {
    const int rows = B * t.n;
    const int chunks = pick_chunks(rows, V);
    const size_t parts = (size_t)rows * chunks;
    float* pv = reinterpret_cast<float*>(ws);
    int* pi = reinterpret_cast<int*>(reinterpret_cast<char*>(ws) + align256(parts * 4));
    hipLaunchKernelGGL(k_argmax_part, dim3((unsigned)parts), dim3(BLOCK), 0, s, logits, V, chunks, pv, pi);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t per_head = (size_t)2 * (K + 1) * hd * (dt == 0 ? 4 : 2);
    const size_t lds = per_head > (size_t)kCompactLds ? per_head : (size_t)kCompactLds;
    if (dt == 0)
        hipLaunchKernelGGL(k_accept<float>, dim3(B), dim3(BLOCK), lds, s, t, K, Hkv, hd, Lcap, chunks, pv, pi,
                           nullptr, tree_tok, reinterpret_cast<float*>(Kc), reinterpret_cast<float*>(Vc), lens,
                           accept_len, path, next_tok, compact_src);
    else
        hipLaunchKernelGGL(k_accept<uint16_t>, dim3(B), dim3(BLOCK), lds, s, t, K, Hkv, hd, Lcap, chunks, pv, pi,
                           nullptr, tree_tok, reinterpret_cast<uint16_t*>(Kc), reinterpret_cast<uint16_t*>(Vc), lens,
                           accept_len, path, next_tok, compact_src);
    return hipGetLastError();
}

hipError_t accept_tokens_launch(const DevTree& t, int dt, int B, int K, int Hkv, int hd, int Lcap,
                                const int32_t* target_tok, const int32_t* tree_tok, void* Kc, void* Vc,
                                int32_t* lens, int32_t* accept_len, int32_t* path, int32_t* next_tok,
                                int32_t* compact_src, hipStream_t s) {
    const size_t per_head = (size_t)2 * (K + 1) * hd * (dt == 0 ? 4 : 2);
    const size_t lds = per_head > (size_t)kCompactLds ? per_head : (size_t)kCompactLds;
    if (dt == 0)
        hipLaunchKernelGGL(k_accept<float>, dim3(B), dim3(BLOCK), lds, s, t, K, Hkv, hd, Lcap, 0, nullptr, nullptr,
                           target_tok, tree_tok, reinterpret_cast<float*>(Kc), reinterpret_cast<float*>(Vc), lens,
                           accept_len, path, next_tok, compact_src);
    else
        hipLaunchKernelGGL(k_accept<uint16_t>, dim3(B), dim3(BLOCK), lds, s, t, K, Hkv, hd, Lcap, 0, nullptr, nullptr,
                           target_tok, tree_tok, reinterpret_cast<uint16_t*>(Kc), reinterpret_cast<uint16_t*>(Vc),
                           lens, accept_len, path, next_tok, compact_src);
    return hipGetLastError();
}
