// Draft heads on the hidden state, reduced straight to per-head top-k lists.
//
// "Medusa heads versus separate draft model", sections "What each one is" and
// "Cost per step": a head is a residual block h' = h + SiLU(W h + b) (W is
// d x d) followed by the head's own d x V vocabulary projection, and at batch
// 1 its cost is the bytes it reads. "Trees": the step keeps only the best few
// candidates of each head. Hydra (abstract; study.space summary): each head
// also sees the token speculated before it, x = [h ; E[parent token]] with W
// of size d x 2d.
//
// GEMV path, for a handful of rows (M <= 4 per pass). Every weight row is
// streamed from HBM exactly once per pass with 16-byte non-temporal loads
// (64 lanes x 16 B = 1 KiB per wave instruction, fully coalesced); the
// activations sit in LDS as float32; each wave streams RPW = 2 rows at a time
// and unrolls the column loop 8 deep, so 16 loads are outstanding per wave.
// (Measured on MI355X at the 70B shape: 2 x 8 and 1 x 16 reach 6.9 TB/s,
// 4 x 4 6.8 TB/s; plain loads instead of non-temporal ones lose 7%.) The dot
// products end in a butterfly reduction that leaves the same bits in every
// lane, so the top-k update is wave-uniform: lanes 0..k-1 hold the sorted
// list in registers and an insertion is one ballot plus one shift. Logits are
// never written; the waves of a block merge their k best (value, index) pairs
// in LDS, each block leaves one list, and a merge kernel reduces the lists of
// all blocks of a head.
#include <math.h>

#include <algorithm>

#include "md_internal.h"
#include "md_sync.h"
#include "md_wave.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int MD_MAX_TOPK_DEV = 16;
constexpr int RPW = 2;     // weight rows in flight per wave
constexpr int UNROLL = 8;  // column steps per loop iteration (RPW x UNROLL loads in flight)
constexpr int BLOCK = 256;
constexpr int NWAVE = BLOCK / MD_WAVE;

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float ldf(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ldf(const uint16_t* p, int64_t i) { return __uint_as_float((uint32_t)p[i] << 16); }

// 16 bytes of weights: loaded raw (non-temporal), widened to float32 at use.
template <typename T>
struct Chunk;
template <>
struct Chunk<uint16_t> {
    static constexpr int N = 8;
    typedef u32x4 Raw;
    __device__ __forceinline__ static Raw load(const uint16_t* p) {
        return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    }
    __device__ __forceinline__ static float at(const Raw& v, int e) {
        const uint32_t w = e < 2 ? v.x : (e < 4 ? v.y : (e < 6 ? v.z : v.w));
        return (e & 1) ? bf_hi(w) : bf_lo(w);
    }
};
template <>
struct Chunk<float> {
    static constexpr int N = 4;
    typedef f32x4 Raw;
    __device__ __forceinline__ static Raw load(const float* p) {
        return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    }
    __device__ __forceinline__ static float at(const Raw& v, int e) {
        return e == 0 ? v.x : (e == 1 ? v.y : (e == 2 ? v.z : v.w));
    }
};

// VEC consecutive float32 activations from LDS (16-byte aligned).
template <int VEC>
__device__ __forceinline__ void lds_vec(const float* p, float (&x)[VEC]) {
#pragma unroll
    for (int e = 0; e < VEC; e += 4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(p + e);
        x[e] = v.x;
        x[e + 1] = v.y;
        x[e + 2] = v.z;
        x[e + 3] = v.w;
    }
}

// 8 consecutive activations (16-byte aligned) widened to float32.
__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(p);
    v[0] = bf_lo(w.x);
    v[1] = bf_hi(w.x);
    v[2] = bf_lo(w.y);
    v[3] = bf_hi(w.y);
    v[4] = bf_lo(w.z);
    v[5] = bf_hi(w.z);
    v[6] = bf_lo(w.w);
    v[7] = bf_hi(w.w);
}
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    v[0] = a.x;
    v[1] = a.y;
    v[2] = a.z;
    v[3] = a.w;
    v[4] = b.x;
    v[5] = b.y;
    v[6] = b.z;
    v[7] = b.w;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, MD_WAVE);
    return v;
}

// Total order of candidates: larger value first, equal values by lower index.
__device__ __forceinline__ bool ranks_above(float v, int i, float w, int j) { return v > w || (v == w && i < j); }

// Sorted list in lanes 0..k-1 (lv, li); insert the wave-uniform candidate (x, xi).
__device__ __forceinline__ void list_insert(float& lv, int& li, float x, int xi, int k, int lane) {
    const bool above = lane < k && ranks_above(lv, li, x, xi);
    const int pos = __popcll(__ballot(above));
    if (pos >= k) return;
    const float pv = __shfl_up(lv, 1, MD_WAVE);
    const int pi = __shfl_up(li, 1, MD_WAVE);
    if (lane == pos) {
        lv = x;
        li = xi;
    } else if (lane > pos && lane < k) {
        lv = pv;
        li = pi;
    }
}

// acc[rr][m] (per lane, partial) = sum over this lane's columns of
// row(r + rr)[c] * xs[m][c]; rows past nvalid repeat the last valid row.
template <typename T, int MR>
__device__ __forceinline__ void rows_dot(const T* __restrict__ base, int64_t stride, int r, int nvalid,
                                         const float* __restrict__ xs, int ncols, int lane,
                                         float (&acc)[RPW][MR]) {
    typedef Chunk<T> C;
    constexpr int VEC = C::N;
    constexpr int STEP = MD_WAVE * VEC;
    const T* rp[RPW];
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
        rp[rr] = base + (int64_t)(r + (rr < nvalid ? rr : nvalid - 1)) * stride;
#pragma unroll
        for (int m = 0; m < MR; ++m) acc[rr][m] = 0.f;
    }
    int c = lane * VEC;
    for (; c + (UNROLL - 1) * STEP < ncols; c += UNROLL * STEP) {
        typename C::Raw w[UNROLL][RPW];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
#pragma unroll
            for (int rr = 0; rr < RPW; ++rr) w[u][rr] = C::load(rp[rr] + c + u * STEP);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                float x[VEC];
                lds_vec<VEC>(xs + m * ncols + c + u * STEP, x);
#pragma unroll
                for (int rr = 0; rr < RPW; ++rr)
#pragma unroll
                    for (int e = 0; e < VEC; ++e) acc[rr][m] = fmaf(C::at(w[u][rr], e), x[e], acc[rr][m]);
            }
        }
    }
    for (; c < ncols; c += STEP) {
        typename C::Raw w[RPW];
#pragma unroll
        for (int rr = 0; rr < RPW; ++rr) w[rr] = C::load(rp[rr] + c);
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            float x[VEC];
            lds_vec<VEC>(xs + m * ncols + c, x);
#pragma unroll
            for (int rr = 0; rr < RPW; ++rr)
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc[rr][m] = fmaf(C::at(w[rr], e), x[e], acc[rr][m]);
        }
    }
}

// Where a row's activation comes from.
struct RowSrc {
    int kind;  // 0: x = h[m]; 1 (Hydra): x = [h[b] ; E[tok(parent)]]
    int P;     // Hydra: rows per request at this level
    int N;     // tree nodes
    int V;     // vocabulary (token range for the E gather)
    int8_t parents[64];
    const void* h;
    const void* E;
    const int32_t* root_tok;
    const int32_t* tree_tok;
};

struct KK {
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

// hres[hh][m][r] = x_m[r] + SiLU(sum_c W[head0+hh][r][c] x_m[c] + b[head0+hh][r])
template <typename T, int MR>
// With hhi (bf16 only, for the matrix-core vocabulary kernels) h' is also
// stored split as hi = bf16(h'), lo = bf16(h' - hi), and block 0 of the
// first pass sets the nh * M row bounds those kernels keep to bound_init.
__global__ __launch_bounds__(BLOCK, 4) void k_residual(const T* __restrict__ W, const T* __restrict__ bias, RowSrc src,
                                                    int M, int m0, int d, int din, int nh, int head0,
                                                    float* __restrict__ hres, float* __restrict__ hres_out,
                                                    uint16_t* __restrict__ hhi, uint16_t* __restrict__ hlo,
                                                    int* __restrict__ bound, int bound_init) {
    extern __shared__ __align__(16) float xs[];  // [MR][din]
    const int mr = min(MR, M - m0);
    const T* h = reinterpret_cast<const T*>(src.h);
    if (bound && m0 == 0 && blockIdx.x == 0)
        for (int j = threadIdx.x; j < nh * M; j += BLOCK) bound[j] = bound_init;
    // 8 activations per 16-byte (bf16) or two 16-byte (f32) loads; d % 8 == 0,
    // so a chunk never straddles the h / E boundary of a Hydra row
    const int nch = MR * din / 8;
    for (int i = threadIdx.x; i < nch; i += BLOCK) {
        const int e0 = i * 8;
        const int mm = e0 / din, c = e0 - (e0 / din) * din;
        float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (mm < mr) {
            const int m = m0 + mm;
            const T* srcp = nullptr;
            if (src.kind == 0) {
                srcp = h + (int64_t)m * d + c;
            } else {
                const int b = m / src.P, j = m - (m / src.P) * src.P;
                if (c < d) {
                    srcp = h + (int64_t)b * d + c;
                } else {
                    const int p = src.parents[j];
                    const int tok = p == 0 ? src.root_tok[b] : src.tree_tok[(int64_t)b * src.N + p];
                    // a token outside the vocabulary (e.g. a -1 left by a failed
                    // lookup) reads as a zero embedding instead of stray memory
                    if (tok >= 0 && tok < src.V) srcp = reinterpret_cast<const T*>(src.E) + (int64_t)tok * d + (c - d);
                }
            }
            if (srcp) load8(srcp, v);
        }
        *reinterpret_cast<f32x4*>(xs + e0) = f32x4{v[0], v[1], v[2], v[3]};
        *reinterpret_cast<f32x4*>(xs + e0 + 4) = f32x4{v[4], v[5], v[6], v[7]};
    }
    __syncthreads();

    const int lane = threadIdx.x & (MD_WAVE - 1);
    const int gw = blockIdx.x * NWAVE + (threadIdx.x >> 6);
    const int tw = gridDim.x * NWAVE;
    const int R = nh * d;
    const int r0 = (int)((int64_t)R * gw / tw), r1 = (int)((int64_t)R * (gw + 1) / tw);
    const T* Wb = W + (int64_t)head0 * d * din;
    for (int r = r0; r < r1; r += RPW) {
        const int nv = min(RPW, r1 - r);
        float acc[RPW][MR];
        rows_dot<T, MR>(Wb, din, r, nv, xs, din, lane, acc);
#pragma unroll
        for (int rr = 0; rr < RPW; ++rr) {
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                const float s = wave_sum(acc[rr][m]);
                if (rr < nv && m < mr && lane == 0) {
                    const int row = r + rr, hh = row / d, ri = row - (row / d) * d;
                    const float z = s + (bias ? ldf(bias, (int64_t)(head0 + hh) * d + ri) : 0.f);
                    const float hv = xs[m * din + ri] + z / (1.f + expf(-z));
                    const int64_t o = ((int64_t)hh * M + m0 + m) * d + ri;
                    hres[o] = hv;
                    if (hres_out) hres_out[o] = hv;
                    if (hhi) {
                        const __bf16 hb = (__bf16)hv;
                        hhi[o] = __builtin_bit_cast(uint16_t, hb);
                        hlo[o] = __builtin_bit_cast(uint16_t, (__bf16)(hv - (float)hb));
                    }
                }
            }
        }
    }
}

// Per wave: the k best logits of U[head0+hh] hres[hh][m] over the wave's rows.
// With one projection shared by the heads (Mh > 0) there is a single U and
// row m of hres ([heads][Mh][d] read as [M][d]) belongs to head m / Mh,
// whose top-k width it takes. NW waves per block share one copy of the MR
// rows of h' in LDS (4 rows of d = 8,192 take 128 KB, so more waves per block
// is the only way to more waves per CU). LOGITS: every logit goes to
// logits_out [row][Ktot][V] instead (sampled decoding needs the heads' whole
// distributions), and no lists are kept.
template <typename T, int MR, int NW, bool LOGITS = false>
__global__ __launch_bounds__(NW * MD_WAVE) void k_vocab_topk(const T* __restrict__ U, const float* __restrict__ hres,
                                                      int M, int m0, int d, int V, int nh, int head0,
                                                      int wg_per_head, KK kk, int kmax, int Mh,
                                                      float* __restrict__ part_val, int* __restrict__ part_idx,
                                                      float* __restrict__ logits_out = nullptr, int Ktot = 0) {
    extern __shared__ __align__(16) float xs[];  // [MR][d]; later the wave lists
    const int hh = blockIdx.x / wg_per_head;
    const int wgi = blockIdx.x - hh * wg_per_head;
    if (hh >= nh) return;
    const int mr = min(MR, M - m0);
    for (int i = threadIdx.x; i < MR * d / 4; i += NW * MD_WAVE) {
        const int e0 = i * 4;
        const int mm = e0 / d, c = e0 - (e0 / d) * d;
        *reinterpret_cast<f32x4*>(xs + e0) =
            mm < mr ? *reinterpret_cast<const f32x4*>(hres + ((int64_t)hh * M + m0 + mm) * d + c)
                    : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    __syncthreads();

    const int lane = threadIdx.x & (MD_WAVE - 1);
    const int wih = wgi * NW + (threadIdx.x >> 6);
    const int wph = wg_per_head * NW;
    const int r0 = (int)((int64_t)V * wih / wph), r1 = (int)((int64_t)V * (wih + 1) / wph);
    int km[MR];  // top-k width of each row
#pragma unroll
    for (int m = 0; m < MR; ++m) km[m] = kk.at(Mh > 0 ? min((m0 + m) / Mh, 7) : hh);
    const T* Uh = U + (int64_t)(head0 + hh) * V * d;

    float lv[MR], tv[MR];
    int li[MR], ti[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        lv[m] = -INFINITY;
        tv[m] = -INFINITY;
        li[m] = INT_MAX;
        ti[m] = INT_MAX;
    }
    for (int r = r0; r < r1; r += RPW) {
        const int nv = min(RPW, r1 - r);
        float acc[RPW][MR];
        rows_dot<T, MR>(Uh, d, r, nv, xs, d, lane, acc);
#pragma unroll
        for (int rr = 0; rr < RPW; ++rr) {
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                const float s = wave_sum(acc[rr][m]);
                if constexpr (LOGITS) {
                    if (rr < nv && m < mr && lane == 0) {
                        const int mv = m0 + m;
                        const int head = Mh > 0 ? mv / Mh : head0 + hh;
                        const int row = Mh > 0 ? mv - head * Mh : mv;
                        logits_out[((int64_t)row * Ktot + head) * V + r + rr] = s;
                    }
                } else if (rr < nv && m < mr && ranks_above(s, r + rr, tv[m], ti[m])) {
                    list_insert(lv[m], li[m], s, r + rr, km[m], lane);
                    tv[m] = __shfl(lv[m], km[m] - 1, MD_WAVE);
                    ti[m] = __shfl(li[m], km[m] - 1, MD_WAVE);
                }
            }
        }
    }
    if constexpr (LOGITS) return;
    // merge the block's wave lists in LDS (over h', now dead); one list per
    // block goes to memory
    __syncthreads();
    float* sv = xs;                                        // [MR][NW][64]
    int* si = reinterpret_cast<int*>(xs + MR * NW * MD_WAVE);  // [MR][NW][64]
    const int wv = threadIdx.x >> 6;
#pragma unroll
    for (int m = 0; m < MR; ++m) {
        sv[(m * NW + wv) * MD_WAVE + lane] = lane < km[m] ? lv[m] : -INFINITY;
        si[(m * NW + wv) * MD_WAVE + lane] = lane < km[m] ? li[m] : INT_MAX;
    }
    __syncthreads();
    // wave m merges the lists of activation row m (the rows in parallel)
    static_assert(NW >= MR, "one wave per activation row");
    const int m = wv;
    if (m >= mr) return;
    const int k = kk.at(Mh > 0 ? min((m0 + m) / Mh, 7) : hh);
    float bv = -INFINITY, btv = -INFINITY;
    int bi = INT_MAX, bti = INT_MAX;
    for (int w2 = 0; w2 < NW; ++w2) {
        const float cv = sv[(m * NW + w2) * MD_WAVE + lane];
        const int ci = si[(m * NW + w2) * MD_WAVE + lane];
        uint64_t bm = __ballot(lane < k && ranks_above(cv, ci, btv, bti));
        while (bm) {
            const int src = __ffsll((long long)bm) - 1;
            bm &= bm - 1;
            const float x = __shfl(cv, src, MD_WAVE);
            const int xi = __shfl(ci, src, MD_WAVE);
            if (ranks_above(x, xi, btv, bti)) {
                list_insert(bv, bi, x, xi, k, lane);
                btv = __shfl(bv, k - 1, MD_WAVE);
                bti = __shfl(bi, k - 1, MD_WAVE);
            }
        }
    }
    if (lane < kmax) {
        const int64_t o = (((int64_t)hh * M + m0 + m) * wg_per_head + wgi) * kmax + lane;
        part_val[o] = bv;
        part_idx[o] = bi;
    }
}

// The k-way merge of nlists sorted lists of k (value, index) pairs at
// pv/pi + base + list * kmax into out_idx/out_val (kmax entries, -1 / -inf
// padded past k), by one block of BLOCK threads. Every list is sorted by
// (value desc, index asc); each wave takes k rounds of a wave-wide argmax
// over its lanes' list heads, each round popping the winning list, and one
// wave merges the waves' sorted lists the same way (no block barrier per
// round). Vocabulary indices are unique, so the order is strict and the
// winner unique. LPT lists per thread; LPT = 0 takes any number of lists:
// each thread first folds lists tid, tid + BLOCK, ... into one sorted list of
// its k best. COH: the lists are read with agent-coherent loads (written by
// other blocks of the same launch).
template <bool COH>
__device__ __forceinline__ float lval(const float* p, int64_t i) {
    if constexpr (COH) return md_sync::get(p + i);
    return p[i];
}
template <bool COH>
__device__ __forceinline__ int lidx(const int* p, int64_t i) {
    if constexpr (COH) return md_sync::get(p + i);
    return p[i];
}

// KM: the register lists' length, at least k (4, 8 or 16: a shorter list
// makes each pop of a winner's head cheaper).
template <int LPT, bool COH, int KM = MD_MAX_TOPK_DEV>
__device__ __forceinline__ void merge_lists(const float* __restrict__ part_val, const int* __restrict__ part_idx,
                                            int64_t base, int nlists, int k, int kmax, int32_t* __restrict__ out_idx,
                                            float* __restrict__ out_val) {
    static_assert(KM <= MD_MAX_TOPK_DEV, "no longer than a head's list");
    __shared__ float wl_v[NWAVE][KM];
    __shared__ int wl_i[NWAVE][KM];
    const int tid = threadIdx.x, lane = tid & (MD_WAVE - 1), w = tid >> 6;
    constexpr int NL = LPT > 0 ? LPT : 1;
    float v[NL][KM];
    int ix[NL][KM];
    if constexpr (LPT > 0) {
#pragma unroll
        for (int l = 0; l < LPT; ++l) {
            const int list = tid + BLOCK * l;
#pragma unroll
            for (int j = 0; j < KM; ++j) {
                const bool ok = list < nlists && j < k;
                v[l][j] = ok ? lval<COH>(part_val, base + (int64_t)list * kmax + j) : -INFINITY;
                ix[l][j] = ok ? lidx<COH>(part_idx, base + (int64_t)list * kmax + j) : INT_MAX;
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < KM; ++j) {
            v[0][j] = -INFINITY;
            ix[0][j] = INT_MAX;
        }
        for (int list = tid; list < nlists; list += BLOCK) {
            for (int j = 0; j < k; ++j) {
                const float cv = lval<COH>(part_val, base + (int64_t)list * kmax + j);
                const int ci = lidx<COH>(part_idx, base + (int64_t)list * kmax + j);
                // a sorted list: once an entry misses this thread's KM best, so do the rest
                if (!ranks_above(cv, ci, v[0][KM - 1], ix[0][KM - 1])) break;
#pragma unroll
                for (int q = KM - 1; q >= 0; --q) {  // insertion; v[0][q - 1] is read before it moves
                    if (!ranks_above(cv, ci, v[0][q], ix[0][q])) continue;
                    if (q > 0 && ranks_above(cv, ci, v[0][q - 1], ix[0][q - 1])) {
                        v[0][q] = v[0][q - 1];
                        ix[0][q] = ix[0][q - 1];
                    } else {
                        v[0][q] = cv;
                        ix[0][q] = ci;
                    }
                }
            }
        }
    }
    // Each wave first pops its own k best from its lanes' lists (no block
    // barrier per round), then wave 0 merges the NWAVE sorted wave lists:
    // NWAVE * k <= 64 candidates, one per lane.
    for (int r = 0; r < k; ++r) {
        float bv = v[0][0];
        int bi = ix[0][0], bo = tid * NL;
#pragma unroll
        for (int l = 1; l < NL; ++l)
            if (ranks_above(v[l][0], ix[l][0], bv, bi)) {
                bv = v[l][0];
                bi = ix[l][0];
                bo = tid * NL + l;
            }
        md_wave::wave_argmax(bv, bi, bo);
        if (lane == 0) {
            wl_v[w][r] = bv;
            wl_i[w][r] = bi;
        }
        if (bo / NL == tid) {  // pop the winning list's head
            const int lw = bo - tid * NL;
#pragma unroll
            for (int l = 0; l < NL; ++l) {
                if (l != lw) continue;
#pragma unroll
                for (int j = 0; j + 1 < KM; ++j) {
                    v[l][j] = v[l][j + 1];
                    ix[l][j] = ix[l][j + 1];
                }
                v[l][KM - 1] = -INFINITY;
                ix[l][KM - 1] = INT_MAX;
            }
        }
    }
    __syncthreads();
    if (w != 0) return;
    static_assert(NWAVE * KM <= MD_WAVE, "one wave list entry per lane");
    float cv = lane < NWAVE * k ? wl_v[lane / k][lane % k] : -INFINITY;
    int ci = lane < NWAVE * k ? wl_i[lane / k][lane % k] : INT_MAX;
    float ov = -INFINITY;
    int oi = INT_MAX;
    for (int r = 0; r < k; ++r) {
        float bv = cv;
        int bi = ci;
        md_wave::wave_argmax(bv, bi);
        if (lane == r) {
            ov = bv;
            oi = bi;
        }
        if (ci == bi) {  // indices are unique: exactly the winner drops out
            cv = -INFINITY;
            ci = INT_MAX;
        }
    }
    if (lane < kmax) {
        const bool ok = lane < k && oi != INT_MAX;
        out_idx[lane] = ok ? oi : -1;
        out_val[lane] = ok ? ov : -INFINITY;
    }
}

// One block per (row m, head slot hh): the k best of the head are the k-way
// merge of the sorted lists every block of the vocabulary kernel left.
template <int LPT, int KM>
__global__ __launch_bounds__(BLOCK) void k_topk_merge(const float* __restrict__ part_val,
                                                      const int* __restrict__ part_idx, int M, int nh, int nlists,
                                                      KK kk, int kmax, int32_t* __restrict__ topk_idx,
                                                      float* __restrict__ topk_val) {
    const int m = blockIdx.x / nh, hh = blockIdx.x - (blockIdx.x / nh) * nh;
    const int64_t base = ((int64_t)hh * M + m) * nlists * kmax;
    const int64_t o = ((int64_t)m * nh + hh) * kmax;
    merge_lists<LPT, false, KM>(part_val, part_idx, base, nlists, kk.at(hh), kmax, topk_idx + o, topk_val + o);
}

// ---- one launch for the heads of one row (Medusa, bf16) ----
//
// The residual blocks, the vocabulary projections, the per-head top-k and
// their k-way merge in a single launch, so the 537 MB of W (70B shape) stream
// in the same kernel as the 8.4 GB of U instead of a short kernel of their
// own, and the merge needs no launch. Block group j (wg blocks) first
// computes h'_j: its waves split the d rows of W[j] as the residual kernel's
// waves split them (same sums, bit for bit). Once every block of the group
// has stored its share, each block loads h'_j and streams its share of U[j]
// exactly as k_vocab_topk does, and the group's first block merges the
// group's lists.
//
// Blocks of a group meet through per-block flag words holding a token
// unique to the launch (md_sync.h): a block writes its share of h' (or its
// list) with agent-coherent stores and raises its flag once they have
// completed; a reader that sees every flag of its group loads the data with
// agent-coherent loads, so no cache write-back or invalidate is needed.
// Every wait is bounded: a block that gives up on its group's h' computes
// all of h'_j itself (reading W[j] alone: slow, the same result); a group
// leader that gives up on the lists writes -1 indices.
constexpr int kSpinRes = 1 << 16;    // ~30 ms of polling before computing h' alone
constexpr int kSpinLists = 1 << 19;  // ~250 ms of polling before giving up the merge
struct SpinLimits {
    int res, lists;  // polls of the two bounded waits
};

__global__ __launch_bounds__(BLOCK) void k_heads_fused(const uint16_t* __restrict__ W,
                                                       const uint16_t* __restrict__ bias,
                                                       const uint16_t* __restrict__ h, const uint16_t* __restrict__ U,
                                                       int d, int V, int nh, int wg, KK kk, int kmax, uint64_t token,
                                                       SpinLimits spin,
                                                       float* __restrict__ hres, float* __restrict__ hres_out,
                                                       float* __restrict__ part_val, int* __restrict__ part_idx,
                                                       uint64_t* __restrict__ flags_res,
                                                       uint64_t* __restrict__ flags_list,
                                                       int32_t* __restrict__ topk_idx, float* __restrict__ topk_val) {
    extern __shared__ __align__(16) float xs[];  // [d]: h, then h'_j, then the wave lists
    const int hh = blockIdx.x / wg, wgi = blockIdx.x - (blockIdx.x / wg) * wg;
    if (hh >= nh) return;
    const int tid = threadIdx.x, lane = tid & (MD_WAVE - 1), wv = tid >> 6;
    for (int i = tid; i < d / 8; i += BLOCK) {
        float v[8];
        load8(h + 8 * i, v);
        *reinterpret_cast<f32x4*>(xs + 8 * i) = f32x4{v[0], v[1], v[2], v[3]};
        *reinterpret_cast<f32x4*>(xs + 8 * i + 4) = f32x4{v[4], v[5], v[6], v[7]};
    }
    __syncthreads();

    // this block's share of h'_hh
    float* hres_h = hres + (int64_t)hh * d;
    {
        const int gw = wgi * NWAVE + wv, tw = wg * NWAVE;
        const int r0 = (int)((int64_t)d * gw / tw), r1 = (int)((int64_t)d * (gw + 1) / tw);
        const uint16_t* Wh = W + (int64_t)hh * d * d;
        // lane j keeps the sum of row r0 + j; the epilogue and its stores come
        // after the last row, so no store's completion holds up the next
        // rows' loads (loads and stores share one counter)
        float mine = 0.f;
        for (int r = r0; r < r1; r += RPW) {
            const int nv = min(RPW, r1 - r);
            float acc[RPW][1];
            rows_dot<uint16_t, 1>(Wh, d, r, nv, xs, d, lane, acc);
#pragma unroll
            for (int rr = 0; rr < RPW; ++rr) {
                const float sum = wave_sum(acc[rr][0]);
                if (rr < nv && lane == ((r - r0 + rr) & (MD_WAVE - 1))) mine = sum;
            }
        }
        // a wave's share is at most 64 rows (the host takes this path only then)
        if (r0 + lane < r1) {
            const int ri = r0 + lane;
            const float z = mine + (bias ? ldf(bias, (int64_t)hh * d + ri) : 0.f);
            const float hv = xs[ri] + z / (1.f + expf(-z));
            md_sync::put(hres_h + ri, hv);
            if (hres_out) hres_out[(int64_t)hh * d + ri] = hv;
        }
    }
    md_sync::raise_flag(flags_res + blockIdx.x, token);

    // h'_hh once the whole group has stored it (h in LDS is no longer read)
    if (md_sync::all_flags<BLOCK>(flags_res + (int64_t)hh * wg, wg, token, spin.res)) {
        for (int i = tid; i < d / 2; i += BLOCK) {
            const uint64_t v = md_sync::get(reinterpret_cast<const uint64_t*>(hres_h) + i);
            xs[2 * i] = __uint_as_float((uint32_t)v);
            xs[2 * i + 1] = __uint_as_float((uint32_t)(v >> 32));
        }
    } else {
        // the group did not finish in time: every row of h'_hh from W and h in
        // memory, in the same order of sums
        const uint16_t* Wh = W + (int64_t)hh * d * d;
        for (int ri = wv; ri < d; ri += NWAVE) {
            const uint16_t* wr = Wh + (int64_t)ri * d;
            float acc = 0.f;
            for (int c = lane * 8; c < d; c += MD_WAVE * 8) {
                float wv8[8], hv8[8];
                load8(wr + c, wv8);
                load8(h + c, hv8);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc = fmaf(wv8[e], hv8[e], acc);
            }
            const float sum = wave_sum(acc);
            if (lane == 0) {
                const float z = sum + (bias ? ldf(bias, (int64_t)hh * d + ri) : 0.f);
                xs[ri] = ldf(h, ri) + z / (1.f + expf(-z));
            }
        }
    }
    __syncthreads();

    // this block's share of the vocabulary rows, as k_vocab_topk<bf16, 1, 4>
    const int k = kk.at(hh);
    float lv = -INFINITY, tv = -INFINITY;
    int li = INT_MAX, ti = INT_MAX;
    auto take = [&](int r, int nv, const float (&acc)[RPW][1]) {
#pragma unroll
        for (int rr = 0; rr < RPW; ++rr) {
            const float sum = wave_sum(acc[rr][0]);
            if (rr < nv && ranks_above(sum, r + rr, tv, ti)) {
                list_insert(lv, li, sum, r + rr, k, lane);
                tv = __shfl(lv, k - 1, MD_WAVE);
                ti = __shfl(li, k - 1, MD_WAVE);
            }
        }
    };
    const int wih = wgi * NWAVE + wv, wph = wg * NWAVE;
    const int v0 = (int)((int64_t)V * wih / wph), v1 = (int)((int64_t)V * (wih + 1) / wph);
    const uint16_t* Uh = U + (int64_t)hh * V * d;
    for (int r = v0; r < v1; r += RPW) {
        const int nv = min(RPW, v1 - r);
        float acc[RPW][1];
        rows_dot<uint16_t, 1>(Uh, d, r, nv, xs, d, lane, acc);
        take(r, nv, acc);
    }
    // the block's list: wave 0 merges the wave lists in LDS (over h', now dead)
    __syncthreads();
    float* sv = xs;                                           // [NWAVE][64]
    int* si = reinterpret_cast<int*>(xs + NWAVE * MD_WAVE);  // [NWAVE][64]
    sv[wv * MD_WAVE + lane] = lane < k ? lv : -INFINITY;
    si[wv * MD_WAVE + lane] = lane < k ? li : INT_MAX;
    __syncthreads();
    if (wv == 0) {
        float bv = -INFINITY, btv = -INFINITY;
        int bi = INT_MAX, bti = INT_MAX;
        for (int w2 = 0; w2 < NWAVE; ++w2) {
            const float cv = sv[w2 * MD_WAVE + lane];
            const int ci = si[w2 * MD_WAVE + lane];
            uint64_t bm = __ballot(lane < k && ranks_above(cv, ci, btv, bti));
            while (bm) {
                const int src = __ffsll((long long)bm) - 1;
                bm &= bm - 1;
                const float x = __shfl(cv, src, MD_WAVE);
                const int xi = __shfl(ci, src, MD_WAVE);
                if (ranks_above(x, xi, btv, bti)) {
                    list_insert(bv, bi, x, xi, k, lane);
                    btv = __shfl(bv, k - 1, MD_WAVE);
                    bti = __shfl(bi, k - 1, MD_WAVE);
                }
            }
        }
        if (lane < kmax) {
            const int64_t o = ((int64_t)hh * wg + wgi) * kmax + lane;
            md_sync::put(part_val + o, bv);
            md_sync::put(part_idx + o, bi);
        }
    }
    md_sync::raise_flag(flags_list + blockIdx.x, token);
    if (wgi != 0) return;

    // the group's first block merges the group's wg lists into head hh's top-k
    int32_t* oi = topk_idx + (int64_t)hh * kmax;
    float* ov = topk_val + (int64_t)hh * kmax;
    if (!md_sync::all_flags<BLOCK>(flags_list + (int64_t)hh * wg, wg, token, spin.lists)) {
        if (tid < kmax) {
            oi[tid] = -1;
            ov[tid] = -INFINITY;
        }
        return;
    }
    const int64_t base = (int64_t)hh * wg * kmax;
    if (wg <= BLOCK)
        merge_lists<1, true>(part_val, part_idx, base, wg, k, kmax, oi, ov);
    else if (wg <= 2 * BLOCK)
        merge_lists<2, true>(part_val, part_idx, base, wg, k, kmax, oi, ov);
    else
        merge_lists<0, true>(part_val, part_idx, base, wg, k, kmax, oi, ov);
}

struct Plan {
    int MR;   // rows per residual pass
    int MRv;  // rows per vocabulary pass
    int res_grid;
    int voc_grid;
    int wg_per_head;
    int wph;
    int voc_nw;  // waves per vocabulary block
    size_t res_lds, voc_lds;
};

constexpr size_t kLDS = 160 * 1024;

int pick_mr(int M, int din) {
    int mr = M >= 4 ? 4 : (M >= 2 ? 2 : 1);
    while (mr > 1 && (size_t)mr * din * 4 > kLDS) mr >>= 1;
    return mr;
}

// Resident blocks per CU for a kernel at this dynamic LDS size, capped at 4,
// so that a grid of CUs x this many blocks runs in a single round.
template <typename K>
int resident_blocks(K kernel, size_t lds, int threads = BLOCK) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, lds) != hipSuccess || n < 1) n = 1;
    return n > 4 ? 4 : n;
}

// Waves per vocabulary block for MR rows per pass. Four rows of h' fill
// 128 KB of LDS, one block per CU; 12 waves (3 per SIMD, 170 VGPRs each) beat
// 8 and 16 (16 spills): 5.9 vs 5.1 and 4.9 TB/s on the 70B-shaped shared
// projection.
constexpr int vocab_waves(int mr) { return mr == 4 ? 12 : NWAVE; }

// nh heads over M rows; with a shared projection the vocabulary stage is one
// matrix over nh * M rows.
template <typename T>
Plan make_plan_t(int M, int d, int din, int nh, int shared_u) {
    Plan p;
    const int rows_v = shared_u ? nh * M : M, nh_u = shared_u ? 1 : nh;
    p.MR = pick_mr(M, din);
    p.MRv = pick_mr(rows_v, d);
    p.res_lds = (size_t)p.MR * din * 4;
    p.voc_nw = vocab_waves(p.MRv);
    p.voc_lds = std::max((size_t)p.MRv * d * 4, (size_t)p.MRv * p.voc_nw * MD_WAVE * 8);  // h', then the wave lists
    const int cus = device_cus();
    int rb, vb;
    switch (p.MR) {
        case 4: rb = resident_blocks(k_residual<T, 4>, p.res_lds); break;
        case 2: rb = resident_blocks(k_residual<T, 2>, p.res_lds); break;
        default: rb = resident_blocks(k_residual<T, 1>, p.res_lds);
    }
    switch (p.MRv) {
        case 4: vb = resident_blocks(k_vocab_topk<T, 4, vocab_waves(4)>, p.voc_lds, p.voc_nw * MD_WAVE); break;
        case 2: vb = resident_blocks(k_vocab_topk<T, 2, vocab_waves(2)>, p.voc_lds, p.voc_nw * MD_WAVE); break;
        default: vb = resident_blocks(k_vocab_topk<T, 1, vocab_waves(1)>, p.voc_lds, p.voc_nw * MD_WAVE);
    }
    p.res_grid = cus * rb;
    const int vg = cus * vb;
    p.wg_per_head = vg / nh_u;
    if (p.wg_per_head < 1) p.wg_per_head = 1;
    p.voc_grid = p.wg_per_head * nh_u;
    p.wph = p.wg_per_head * p.voc_nw;
    return p;
}

Plan make_plan(int dt, int M, int d, int din, int nh, int shared_u) {
    return dt == 0 ? make_plan_t<float>(M, d, din, nh, shared_u) : make_plan_t<uint16_t>(M, d, din, nh, shared_u);
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The k-way merge of nlists sorted lists per (row, head).
template <int KM>
void launch_merge_km(int lpt, const float* pv, const int* pi, int M, int nh, int nlists, KK kk, int kmax,
                     int32_t* topk_idx, float* topk_val, hipStream_t s) {
    if (lpt <= 1)
        hipLaunchKernelGGL((k_topk_merge<1, KM>), dim3(M * nh), dim3(BLOCK), 0, s, pv, pi, M, nh, nlists, kk, kmax,
                           topk_idx, topk_val);
    else if (lpt == 2)
        hipLaunchKernelGGL((k_topk_merge<2, KM>), dim3(M * nh), dim3(BLOCK), 0, s, pv, pi, M, nh, nlists, kk, kmax,
                           topk_idx, topk_val);
    else if (lpt <= 4)
        hipLaunchKernelGGL((k_topk_merge<4, KM>), dim3(M * nh), dim3(BLOCK), 0, s, pv, pi, M, nh, nlists, kk, kmax,
                           topk_idx, topk_val);
    else
        hipLaunchKernelGGL((k_topk_merge<0, KM>), dim3(M * nh), dim3(BLOCK), 0, s, pv, pi, M, nh, nlists, kk, kmax,
                           topk_idx, topk_val);
}
hipError_t launch_merge(const float* pv, const int* pi, int M, int nh, int nlists, KK kk, int kmax, int32_t* topk_idx,
                        float* topk_val, hipStream_t s) {
    const int lpt = (nlists + BLOCK - 1) / BLOCK;
    int kbig = 1;  // the largest k of the call's heads
    for (int i = 0; i < nh && i < 8; ++i) kbig = std::max(kbig, kk.v[i]);
    if (kbig <= 4)
        launch_merge_km<4>(lpt, pv, pi, M, nh, nlists, kk, kmax, topk_idx, topk_val, s);
    else if (kbig <= 8)
        launch_merge_km<8>(lpt, pv, pi, M, nh, nlists, kk, kmax, topk_idx, topk_val, s);
    else
        launch_merge_km<16>(lpt, pv, pi, M, nh, nlists, kk, kmax, topk_idx, topk_val, s);
    return hipGetLastError();
}

RowSrc row_src(const HeadsArgs& a, const DevTree* tree) {
    RowSrc src;
    src.kind = a.kind;
    src.P = 1;
    src.N = tree ? tree->n : 0;
    src.V = a.V;
    src.h = a.h;
    src.E = a.E;
    src.root_tok = a.root_tok;
    src.tree_tok = a.tree_tok;
    for (int i = 0; i < 64; ++i) src.parents[i] = 0;
    if (a.kind == 1) {
        const int off = tree->level_off[a.level];
        src.P = tree->level_off[a.level + 1] - off;
        for (int j = 0; j < src.P; ++j) src.parents[j] = tree->lp[off + j];
    }
    return src;
}

template <typename T>
hipError_t launch_typed(const HeadsArgs& a, const DevTree* tree, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    const Plan p = make_plan(a.dt, a.M, a.d, a.din, a.nh, a.shared_u);
    char* ws = reinterpret_cast<char*>(a.ws);
    float* hres = reinterpret_cast<float*>(ws);
    ws += align256((size_t)a.nh * a.M * a.d * 4);
    float* pv = reinterpret_cast<float*>(ws);
    ws += align256((size_t)a.nh * a.M * p.wg_per_head * a.kmax * 4);
    int* pi = reinterpret_cast<int*>(ws);

    const RowSrc src = row_src(a, tree);
    KK kk;
    for (int i = 0; i < 8; ++i) kk.v[i] = i < a.nh ? a.kk[i] : 1;

    const T* W = reinterpret_cast<const T*>(a.W);
    const T* bias = reinterpret_cast<const T*>(a.b);
    const T* U = reinterpret_cast<const T*>(a.U);
    // the logits mode takes the K in the output's layout from the call
    const int ktot = a.logits_k;
    for (int m0 = 0; m0 < a.M; m0 += p.MR) {
        switch (p.MR) {
            case 4:
                hipLaunchKernelGGL((k_residual<T, 4>), dim3(p.res_grid), dim3(BLOCK), p.res_lds, s, W, bias, src, a.M,
                                   m0, a.d, a.din, a.nh, a.head0, hres, a.h_res, nullptr, nullptr, nullptr, 0);
                break;
            case 2:
                hipLaunchKernelGGL((k_residual<T, 2>), dim3(p.res_grid), dim3(BLOCK), p.res_lds, s, W, bias, src, a.M,
                                   m0, a.d, a.din, a.nh, a.head0, hres, a.h_res, nullptr, nullptr, nullptr, 0);
                break;
            default:
                hipLaunchKernelGGL((k_residual<T, 1>), dim3(p.res_grid), dim3(BLOCK), p.res_lds, s, W, bias, src, a.M,
                                   m0, a.d, a.din, a.nh, a.head0, hres, a.h_res, nullptr, nullptr, nullptr, 0);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (ev0) {
        hipError_t e = hipEventRecord(ev0, s);
        if (e != hipSuccess) return e;
    }
    // a shared projection is one matrix over the heads' nh * M rows
    const int rows_v = a.shared_u ? a.nh * a.M : a.M, nh_u = a.shared_u ? 1 : a.nh;
    const int head0_u = a.shared_u ? 0 : a.head0, Mh = a.shared_u ? a.M : 0;
    for (int m0 = 0; m0 < rows_v && a.logits; m0 += p.MRv) {
        switch (p.MRv) {
            case 4:
                hipLaunchKernelGGL((k_vocab_topk<T, 4, vocab_waves(4), true>), dim3(p.voc_grid),
                                   dim3(p.voc_nw * MD_WAVE), p.voc_lds, s, U, hres, rows_v, m0, a.d, a.V, nh_u, head0_u,
                                   p.wg_per_head, kk, a.kmax, Mh, pv, pi, a.logits, ktot);
                break;
            case 2:
                hipLaunchKernelGGL((k_vocab_topk<T, 2, vocab_waves(2), true>), dim3(p.voc_grid),
                                   dim3(p.voc_nw * MD_WAVE), p.voc_lds, s, U, hres, rows_v, m0, a.d, a.V, nh_u, head0_u,
                                   p.wg_per_head, kk, a.kmax, Mh, pv, pi, a.logits, ktot);
                break;
            default:
                hipLaunchKernelGGL((k_vocab_topk<T, 1, vocab_waves(1), true>), dim3(p.voc_grid),
                                   dim3(p.voc_nw * MD_WAVE), p.voc_lds, s, U, hres, rows_v, m0, a.d, a.V, nh_u, head0_u,
                                   p.wg_per_head, kk, a.kmax, Mh, pv, pi, a.logits, ktot);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.logits) return ev1 ? hipEventRecord(ev1, s) : hipSuccess;
    for (int m0 = 0; m0 < rows_v; m0 += p.MRv) {
        switch (p.MRv) {
            case 4:
                hipLaunchKernelGGL((k_vocab_topk<T, 4, vocab_waves(4)>), dim3(p.voc_grid), dim3(p.voc_nw * MD_WAVE),
                                   p.voc_lds, s, U, hres, rows_v,
                                   m0, a.d, a.V, nh_u, head0_u, p.wg_per_head, kk, a.kmax, Mh, pv, pi);
                break;
            case 2:
                hipLaunchKernelGGL((k_vocab_topk<T, 2, vocab_waves(2)>), dim3(p.voc_grid), dim3(p.voc_nw * MD_WAVE),
                                   p.voc_lds, s, U, hres, rows_v,
                                   m0, a.d, a.V, nh_u, head0_u, p.wg_per_head, kk, a.kmax, Mh, pv, pi);
                break;
            default:
                hipLaunchKernelGGL((k_vocab_topk<T, 1, vocab_waves(1)>), dim3(p.voc_grid), dim3(p.voc_nw * MD_WAVE),
                                   p.voc_lds, s, U, hres, rows_v,
                                   m0, a.d, a.V, nh_u, head0_u, p.wg_per_head, kk, a.kmax, Mh, pv, pi);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (ev1) {
        hipError_t e = hipEventRecord(ev1, s);
        if (e != hipSuccess) return e;
    }
    return launch_merge(pv, pi, a.M, a.nh, p.wg_per_head, kk, a.kmax, a.topk_idx, a.topk_val, s);
}

}  // namespace

// One Medusa row (its heads' h' through a shared projection are several
// columns): the GEMV residual streams W at ~5.6 TB/s, where a one-row
// matrix-core residual would stage 128-row tiles for a single column. With
// 4 rows the GEMV's 128 KB of LDS a block leaves one block a CU; the
// matrix-core residual stays there.
bool residual_on_gemv(int dt, int kind, int M, int d, int din, bool op) {
    return dt == 1 && kind == 0 && din == d && op && M == 1;
}

hipError_t residual_gemv_split(const HeadsArgs& a, const DevTree* tree, float* hres, uint16_t* hhi, uint16_t* hlo,
                               int* bound, int bound_init, hipStream_t s) {
    const Plan p = make_plan(a.dt, a.M, a.d, a.din, a.nh, a.shared_u);
    const RowSrc src = row_src(a, tree);
    const uint16_t* W = reinterpret_cast<const uint16_t*>(a.W);
    const uint16_t* bias = reinterpret_cast<const uint16_t*>(a.b);
    switch (p.MR) {  // one pass: residual_on_gemv admits only M <= MR
        case 4:
            hipLaunchKernelGGL((k_residual<uint16_t, 4>), dim3(p.res_grid), dim3(BLOCK), p.res_lds, s, W, bias, src, a.M,
                               0, a.d, a.din, a.nh, a.head0, hres, a.h_res, hhi, hlo, bound, bound_init);
            break;
        case 2:
            hipLaunchKernelGGL((k_residual<uint16_t, 2>), dim3(p.res_grid), dim3(BLOCK), p.res_lds, s, W, bias, src, a.M,
                               0, a.d, a.din, a.nh, a.head0, hres, a.h_res, hhi, hlo, bound, bound_init);
            break;
        default:
            hipLaunchKernelGGL((k_residual<uint16_t, 1>), dim3(p.res_grid), dim3(BLOCK), p.res_lds, s, W, bias, src, a.M,
                               0, a.d, a.din, a.nh, a.head0, hres, a.h_res, hhi, hlo, bound, bound_init);
    }
    return hipGetLastError();
}

size_t heads_fused_ws_bytes(int d, int nh, int kmax);

size_t heads_ws_bytes(int dt, int M, int d, int din, int V, int nh, int kmax, int shared_u, bool op) {
    if (heads_fused_applicable(dt, M, d, din, shared_u, nh)) return heads_fused_ws_bytes(d, nh, kmax);
    if (heads_mfma_applicable(dt, M, d, din, op, shared_u ? nh * M : M))
        return heads_mfma_ws_bytes(M, d, din, V, nh, kmax, shared_u);
    const Plan p = make_plan(dt, M, d, din, nh, shared_u);
    return align256((size_t)nh * M * d * 4) + 2 * align256((size_t)nh * M * p.wg_per_head * kmax * 4);
}

size_t heads_logits_ws_bytes(int M, int d, int nh) { return align256((size_t)nh * M * d * 4); }

hipError_t topk_merge_launch(const float* pv, const int* pi, int M, int nh, int nlists, const int* kk, int kmax,
                             int32_t* idx, float* val, hipStream_t s) {
    KK k;
    for (int i = 0; i < 8; ++i) k.v[i] = i < nh ? kk[i] : 1;
    return launch_merge(pv, pi, M, nh, nlists, k, kmax, idx, val, s);
}

size_t heads_ws_bound(int dt, int M, int d, int din, int V, int nh, int kmax, int shared_u) {
    // with or without an operand-order copy of U
    const size_t mfma =
        heads_mfma_applicable(dt, M, d, din, true, shared_u ? nh * M : M) ? heads_mfma_ws_bytes(M, d, din, V, nh, kmax, shared_u)
                                                                          : 0;
    const size_t lists_max = (size_t)device_cus() * 4;  // blocks per head at most
    size_t gemv = align256((size_t)nh * M * d * 4) + 2 * align256((size_t)nh * M * lists_max * kmax * 4);
    // the fused one-row launch adds two flag words per block
    if (heads_fused_applicable(dt, M, d, din, shared_u, nh)) gemv += 2 * align256((size_t)nh * lists_max * 8);
    return gemv > mfma ? gemv : mfma;
}

namespace {

__global__ void k_widen_bf16(const uint16_t* __restrict__ x, float* __restrict__ y, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) y[i] = __uint_as_float((uint32_t)x[i] << 16);
}

// GEMV path of the target argmax: R rows of hidden states (float32 in LDS)
// against the LM head, k = 1 per row, then the k-way merge.
template <typename T>
hipError_t target_argmax_gemv(int dt, int R, int d, int V, const void* H, const void* Wt, int32_t* tok, float* val,
                              void* ws, hipStream_t s) {
    const Plan p = make_plan(dt, R, d, d, 1, 0);
    char* w = reinterpret_cast<char*>(ws);
    const float* hf = reinterpret_cast<const float*>(H);
    if (dt == 1) {
        float* buf = reinterpret_cast<float*>(w);
        w += align256((size_t)R * d * 4);
        const int64_t n = (int64_t)R * d;
        hipLaunchKernelGGL(k_widen_bf16, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                           reinterpret_cast<const uint16_t*>(H), buf, n);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hf = buf;
    }
    float* pv = reinterpret_cast<float*>(w);
    w += align256((size_t)R * p.wg_per_head * 4);
    int* pi = reinterpret_cast<int*>(w);
    w += align256((size_t)R * p.wg_per_head * 4);
    float* vs = reinterpret_cast<float*>(w);  // values when the caller wants none
    KK kk;
    for (int i = 0; i < 8; ++i) kk.v[i] = 1;
    const T* U = reinterpret_cast<const T*>(Wt);
    for (int m0 = 0; m0 < R; m0 += p.MRv) {
        switch (p.MRv) {
            case 4:
                hipLaunchKernelGGL((k_vocab_topk<T, 4, vocab_waves(4)>), dim3(p.voc_grid), dim3(p.voc_nw * MD_WAVE),
                                   p.voc_lds, s, U, hf, R, m0, d, V, 1, 0, p.wg_per_head, kk, 1, 0, pv, pi);
                break;
            case 2:
                hipLaunchKernelGGL((k_vocab_topk<T, 2, vocab_waves(2)>), dim3(p.voc_grid), dim3(p.voc_nw * MD_WAVE),
                                   p.voc_lds, s, U, hf, R, m0, d, V, 1, 0, p.wg_per_head, kk, 1, 0, pv, pi);
                break;
            default:
                hipLaunchKernelGGL((k_vocab_topk<T, 1, vocab_waves(1)>), dim3(p.voc_grid), dim3(p.voc_nw * MD_WAVE),
                                   p.voc_lds, s, U, hf, R, m0, d, V, 1, 0, p.wg_per_head, kk, 1, 0, pv, pi);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return launch_merge(pv, pi, R, 1, p.wg_per_head, kk, 1, tok, val ? val : vs, s);
}

}  // namespace

size_t target_argmax_ws_bound(int dt, int R, int d, int V) {
    const size_t vals = align256((size_t)R * 4);
    const size_t mfma = argmax_mfma_applicable(dt, R, d, true) ? argmax_mfma_ws_bytes(R, V) + vals : 0;
    const size_t lists_max = (size_t)device_cus() * 4;
    const size_t gemv = (dt == 1 ? align256((size_t)R * d * 4) : 0) + 2 * align256((size_t)R * lists_max * 4) + vals;
    return gemv > mfma ? gemv : mfma;
}

hipError_t target_argmax_launch(int dt, int R, int d, int V, const void* H, const void* Wt, const void* Wt_op,
                                int32_t* tok, float* val, void* ws, hipStream_t s) {
    KK kk;
    for (int i = 0; i < 8; ++i) kk.v[i] = 1;
    if (argmax_mfma_applicable(dt, R, d, Wt_op != nullptr)) {
        float* pv;
        int* pi;
        int nlists;
        hipError_t e = argmax_mfma_launch(R, d, V, H, Wt, Wt_op, ws, s, &pv, &pi, &nlists);
        if (e != hipSuccess) return e;
        float* vs = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + argmax_mfma_ws_bytes(R, V));
        return launch_merge(pv, pi, R, 1, nlists, kk, 1, tok, val ? val : vs, s);
    }
    if (dt == 0) return target_argmax_gemv<float>(dt, R, d, V, H, Wt, tok, val, ws, s);
    return target_argmax_gemv<uint16_t>(dt, R, d, V, H, Wt, tok, val, ws, s);
}

namespace {

struct FusedPlan {
    int wg;     // blocks per head
    size_t lds;
};

FusedPlan fused_plan(int d, int nh) {
    FusedPlan p;
    p.lds = std::max((size_t)d * 4, (size_t)NWAVE * MD_WAVE * 8);
    const int occ = resident_blocks(k_heads_fused, p.lds);
    p.wg = std::max(1, device_cus() * occ / nh);
    return p;
}

struct FusedWs {
    float* hres;
    float* pv;
    int* pi;
    uint64_t *flags_res, *flags_list;
    size_t bytes;
};

FusedWs fused_ws(char* base, int d, int nh, int wg, int kmax) {
    FusedWs L = {};
    size_t off = 0;
    auto take = [&](size_t n) {
        char* q = base ? base + off : nullptr;
        off += align256(n);
        return q;
    };
    const size_t lists = (size_t)nh * wg * kmax * 4, flags = (size_t)nh * wg * 8;
    L.hres = reinterpret_cast<float*>(take((size_t)nh * d * 4));
    L.pv = reinterpret_cast<float*>(take(lists));
    L.pi = reinterpret_cast<int*>(take(lists));
    L.flags_res = reinterpret_cast<uint64_t*>(take(flags));
    L.flags_list = reinterpret_cast<uint64_t*>(take(flags));
    L.bytes = off;
    return L;
}

hipError_t heads_fused_launch(const HeadsArgs& a, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    const FusedPlan p = fused_plan(a.d, a.nh);
    const FusedWs L = fused_ws(reinterpret_cast<char*>(a.ws), a.d, a.nh, p.wg, a.kmax);
    KK kk;
    for (int i = 0; i < 8; ++i) kk.v[i] = i < a.nh ? a.kk[i] : 1;
    hipError_t e;
    if (ev0 && (e = hipEventRecord(ev0, s)) != hipSuccess) return e;
    hipLaunchKernelGGL(k_heads_fused, dim3((unsigned)(a.nh * p.wg)), dim3(BLOCK), p.lds, s,
                       reinterpret_cast<const uint16_t*>(a.W), reinterpret_cast<const uint16_t*>(a.b),
                       reinterpret_cast<const uint16_t*>(a.h), reinterpret_cast<const uint16_t*>(a.U), a.d, a.V, a.nh,
                       p.wg, kk, a.kmax, launch_token(),
                       SpinLimits{a.spin_res >= 0 ? a.spin_res : kSpinRes, a.spin_lists >= 0 ? a.spin_lists : kSpinLists},
                       L.hres, a.h_res, L.pv, L.pi, L.flags_res, L.flags_list,
                       a.topk_idx, a.topk_val);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (ev1 && (e = hipEventRecord(ev1, s)) != hipSuccess) return e;
    return hipSuccess;
}

}  // namespace

// One Medusa row in bf16 through per-head projections: the single fused launch
// (while a wave's share of a head's residual rows is at most 64, one per lane).
bool heads_fused_applicable(int dt, int M, int d, int din, int shared_u, int nh) {
    if (!(dt == 1 && M == 1 && din == d && !shared_u && nh >= 1)) return false;
    const FusedPlan p = fused_plan(d, nh);
    return (d + p.wg * NWAVE - 1) / (p.wg * NWAVE) <= MD_WAVE;
}

size_t heads_fused_ws_bytes(int d, int nh, int kmax) {
    return fused_ws(nullptr, d, nh, fused_plan(d, nh).wg, kmax).bytes;
}

hipError_t heads_launch(const HeadsArgs& a, const DevTree* tree, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1) {
    if (!a.logits && a.kind == 0 && heads_fused_applicable(a.dt, a.M, a.d, a.din, a.shared_u, a.nh))
        return heads_fused_launch(a, s, ev0, ev1);
    if (!a.logits &&
        heads_mfma_applicable(a.dt, a.M, a.d, a.din, a.U_op != nullptr, a.shared_u ? a.nh * a.M : a.M)) {
        // many rows: the two contractions on the matrix cores, then the same k-way merge
        float* pv;
        int* pi;
        int nlists;
        hipError_t e = heads_mfma_launch(a, tree, s, ev0, ev1, &pv, &pi, &nlists);
        if (e != hipSuccess) return e;
        if (nlists == 0) return hipSuccess;  // the certified pass wrote the lists
        KK kk;
        for (int i = 0; i < 8; ++i) kk.v[i] = i < a.nh ? a.kk[i] : 1;
        return launch_merge(pv, pi, a.M, a.nh, nlists, kk, a.kmax, a.topk_idx, a.topk_val, s);
    }
    if (a.dt == 0) return launch_typed<float>(a, tree, s, ev0, ev1);
    return launch_typed<uint16_t>(a, tree, s, ev0, ev1);
}
