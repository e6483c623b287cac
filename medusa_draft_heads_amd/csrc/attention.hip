// Tree-masked attention of every tree node over the KV cache, in one pass.
//
// "Medusa heads versus separate draft model", section "Trees": all branches
// of the candidate tree are verified in one pass under a tree attention mask.
// Node n sees the cached prefix [0, L_b) and the tree slots L_b + j of its own
// root path (j = n or an ancestor of n). The mask is one 64-bit ancestor set
// per node (bit j), never a dense N x N tensor; key index and cache slot
// coincide (slot L_b + j is key L_b + j).
//
// Work split (flash-decoding style, within one GPU): a block owns one
// (request, kv head, tile of QT query rows, range of keys). The query rows of
// a kv head are its Hq/Hkv query heads times the N nodes, so K and V tiles
// staged in LDS serve every query head of the group. Each block keeps an
// online softmax (running max, running sum, unnormalised output) and writes
// them; a combine kernel merges the key ranges by log-sum-exp.
//
// bf16 storage runs on the matrix cores (v_mfma_f32_16x16x32_bf16): a wave
// owns 16 query rows and computes S^T = K Q^T per 16-key block, then
// O^T += V^T P^T. In this orientation a lane keeps one query row (lane % 16)
// in both the score and the output accumulators, so the running max, the
// rescale and the bf16 P operand never leave the lane. K tiles sit in LDS
// row-major (rows padded by 16 B against bank conflicts), V tiles transposed
// (key-contiguous) so the V^T operand is two 8-byte reads. float32 storage
// (small workloads) uses an LDS-tiled FMA kernel.
#include <math.h>

#include "md_internal.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int QT = 16;  // query rows per block (FMA kernel)
constexpr int MQT = 64; // query rows per block (MFMA kernel: 4 waves x 16)
constexpr int MKT = 64; // keys per tile (MFMA kernel)
constexpr int KPAD = 8; // K row padding, bf16 elements
constexpr int VPAD = 4; // V^T row padding, bf16 elements (rows stay 8-byte aligned)
constexpr int KT = 64;  // keys per tile
constexpr int BLOCK = 256;
constexpr int NWAVE = BLOCK / MD_WAVE;
constexpr int ROWS_PER_WAVE = QT / NWAVE;

__device__ __forceinline__ float ldf(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ldf(const uint16_t* p, int64_t i) { return __uint_as_float((uint32_t)p[i] << 16); }

__device__ __forceinline__ void st(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void st(uint16_t* p, int64_t i, float v) {
    uint32_t u = __float_as_uint(v);
    u += 0x7FFFu + ((u >> 16) & 1u);
    p[i] = (uint16_t)(u >> 16);
}

// 16 bytes of K or V into LDS as float32.
__device__ __forceinline__ void load16(const float* src, float* dst) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(src);
    dst[0] = v.x;
    dst[1] = v.y;
    dst[2] = v.z;
    dst[3] = v.w;
}
__device__ __forceinline__ void load16(const uint16_t* src, float* dst) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(src);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        dst[2 * e] = __uint_as_float(w[e] << 16);
        dst[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, MD_WAVE));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, MD_WAVE);
    return v;
}

template <typename T, int HD>
__global__ __launch_bounds__(BLOCK) void k_attn_fma(DevTree t, int Hq, int Hkv, int Lcap, int max_len,
                                                    const T* __restrict__ q, const T* __restrict__ Kc,
                                                    const T* __restrict__ Vc, const int32_t* __restrict__ lens,
                                                    float scale, int splits, int chunk, int qtiles,
                                                    float* __restrict__ po, float* __restrict__ pm,
                                                    float* __restrict__ pl) {
    constexpr int VEC = 16 / sizeof(T);
    constexpr int CPR = HD / VEC;  // 16-byte chunks per key row
    constexpr int PV_COLS = BLOCK < HD ? BLOCK : HD;
    constexpr int PV_ROWS = QT * HD / BLOCK;  // outputs per thread
    __shared__ float Qs[QT][HD];
    __shared__ float Ks[KT][HD + 1];
    __shared__ float Vs[KT][HD];
    __shared__ float Ps[QT][KT];
    __shared__ float alpha_s[QT];
    __shared__ uint64_t anc_s[QT];

    int bid = blockIdx.x;
    const int s = bid % splits;
    bid /= splits;
    const int qt = bid % qtiles;
    bid /= qtiles;
    const int g = bid % Hkv;
    const int b = bid / Hkv;
    const int group = Hq / Hkv;
    const int N = t.n;
    const int rows = N * group;
    const int L = min(max(lens[b], 0), max_len);
    const int nkeys = L + N;
    const int k0 = s * chunk, k1 = min(k0 + chunk, nkeys);
    const int tid = threadIdx.x, lane = tid & (MD_WAVE - 1), w = tid >> 6;
    const int64_t kvbase = ((int64_t)b * Hkv + g) * Lcap;

    for (int i = tid; i < QT * HD; i += BLOCK) {
        const int qi = i / HD, c = i - (i / HD) * HD;
        const int r = qt * QT + qi;
        float v = 0.f;
        if (r < rows) {
            const int n = r / group, h = g * group + (r - (r / group) * group);
            v = ldf(q, (((int64_t)b * N + n) * Hq + h) * HD + c);
        }
        Qs[qi][c] = v;
    }
    if (tid < QT) {
        const int r = qt * QT + tid;
        anc_s[tid] = r < rows ? t.anc[r / group] : 0ull;
    }

    const float scale_log2 = scale * 1.44269504088896340736f;
    float m_i[ROWS_PER_WAVE], l_i[ROWS_PER_WAVE];
#pragma unroll
    for (int j = 0; j < ROWS_PER_WAVE; ++j) {
        m_i[j] = -INFINITY;
        l_i[j] = 0.f;
    }
    float acc[PV_ROWS];
#pragma unroll
    for (int j = 0; j < PV_ROWS; ++j) acc[j] = 0.f;
    const int pc = tid % PV_COLS, pr0 = tid / PV_COLS;

    for (int kt0 = k0; kt0 < k1; kt0 += KT) {
        __syncthreads();
        for (int i = tid; i < KT * CPR; i += BLOCK) {
            const int kk = i / CPR, ch = i - (i / CPR) * CPR;
            const int key = kt0 + kk;
            if (key < k1) {
                load16(Kc + (kvbase + key) * HD + ch * VEC, &Ks[kk][ch * VEC]);
                load16(Vc + (kvbase + key) * HD + ch * VEC, &Vs[kk][ch * VEC]);
            } else {
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    Ks[kk][ch * VEC + e] = 0.f;
                    Vs[kk][ch * VEC + e] = 0.f;
                }
            }
        }
        __syncthreads();
        // scores: wave w owns rows w + NWAVE*j; lane = key within the tile
        const int key = kt0 + lane;
        const bool in_range = key < k1;
#pragma unroll
        for (int j = 0; j < ROWS_PER_WAVE; ++j) {
            const int qi = w + NWAVE * j;
            float sc = 0.f;
#pragma unroll 8
            for (int c = 0; c < HD; ++c) sc = fmaf(Qs[qi][c], Ks[lane][c], sc);
            bool vis = in_range;
            if (vis && key >= L) vis = (anc_s[qi] >> (key - L)) & 1ull;
            sc = vis ? sc * scale_log2 : -INFINITY;
            const float mx = wave_max(sc);
            const float m_new = fmaxf(m_i[j], mx);
            const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_i[j] - m_new);
            const float p = vis ? exp2f(sc - m_new) : 0.f;
            l_i[j] = l_i[j] * alpha + wave_sum(p);
            m_i[j] = m_new;
            Ps[qi][lane] = p;
            if (lane == 0) alpha_s[qi] = alpha;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < PV_ROWS; ++j) {
            const int qi = pr0 + (BLOCK / PV_COLS) * j;
            float a = acc[j] * alpha_s[qi];
#pragma unroll 8
            for (int kk = 0; kk < KT; ++kk) a = fmaf(Ps[qi][kk], Vs[kk][pc], a);
            acc[j] = a;
        }
    }

    // write the unnormalised partial output and the row statistics
#pragma unroll
    for (int j = 0; j < PV_ROWS; ++j) {
        const int qi = pr0 + (BLOCK / PV_COLS) * j;
        const int r = qt * QT + qi;
        if (r < rows) {
            const int n = r / group, h = g * group + (r - (r / group) * group);
            const int64_t row = ((int64_t)b * N + n) * Hq + h;
            po[(row * splits + s) * HD + pc] = acc[j];
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int j = 0; j < ROWS_PER_WAVE; ++j) {
            const int qi = w + NWAVE * j;
            const int r = qt * QT + qi;
            if (r < rows) {
                const int n = r / group, h = g * group + (r - (r / group) * group);
                const int64_t row = ((int64_t)b * N + n) * Hq + h;
                pm[row * splits + s] = m_i[j];
                pl[row * splits + s] = l_i[j];
            }
        }
    }
}


// Value of lane ^ 16 / lane ^ 32. The gfx950 row swaps exchange 16-lane rows
// between two registers; swapping a register with itself leaves the own row
// in one result and the partner row in the other, in an order that depends
// on the row -- so the pair is only combined symmetrically (max, +).
__device__ __forceinline__ float xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
    return a == v ? b : a;
}
__device__ __forceinline__ float xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
    return a == v ? b : a;
}

// Blocks that share one (request, kv head, key range) -- the query tiles of a
// group -- read the same K/V tiles. Workgroups go to the 8 XCDs round-robin
// (block id mod 8), each XCD with its own L2, so the ids of one group are
// spaced by 8: the whole group runs on one XCD and its K/V tiles come from
// HBM once. Ids past the last group exit at once.
__device__ __forceinline__ bool xcd_group_decode(int id, int qtiles, int ngroups, int& group, int& qt) {
    const int x = id & 7, u = id >> 3;
    qt = u % qtiles;
    group = (u / qtiles) * 8 + x;
    return group < ngroups;
}

template <int HD>
__global__ __launch_bounds__(BLOCK, 3) void k_attn_mfma(DevTree t, int Hq, int Hkv, int Lcap, int max_len,
                                                     const uint16_t* __restrict__ q, const uint16_t* __restrict__ Kc,
                                                     const uint16_t* __restrict__ Vc, const int32_t* __restrict__ lens,
                                                     float scale, int splits, int chunk, int qtiles, int ngroups,
                                                     float* __restrict__ po, float* __restrict__ pm,
                                                     float* __restrict__ pl) {
    constexpr int CH = HD / 8;            // 16-byte chunks per key row
    constexpr int KCH = MKT * CH / BLOCK; // K chunks per thread
    constexpr int VIT = (MKT / 4) * CH;   // V items (4 keys x 8 dims)
    __shared__ __align__(16) uint16_t Ks[MKT][HD + KPAD];
    __shared__ __align__(16) uint16_t Vt[HD][MKT + VPAD];

    int grp, qt;
    if (!xcd_group_decode(blockIdx.x, qtiles, ngroups, grp, qt)) return;
    const int s = grp % splits;
    const int g = (grp / splits) % Hkv;
    const int b = grp / (splits * Hkv);
    const int group = Hq / Hkv;
    const int N = t.n;
    const int rows = N * group;
    const int L = min(max(lens[b], 0), max_len);
    const int nkeys = L + N;
    const int k0 = s * chunk, k1 = min(k0 + chunk, nkeys);
    const int tid = threadIdx.x, lane = tid & (MD_WAVE - 1), w = tid >> 6;
    const int g4 = lane >> 4, c16 = lane & 15;
    const int64_t kvbase = ((int64_t)b * Hkv + g) * Lcap;

    // this lane's query row (the N index of both products)
    const int r = qt * MQT + w * 16 + c16;
    const bool rvalid = r < rows;
    const int node = rvalid ? r / group : 0;
    const int h = g * group + (rvalid ? r - (r / group) * group : 0);
    const uint64_t anc = rvalid ? t.anc[node] : 0ull;
    const int64_t qrow = (((int64_t)b * N + node) * Hq + h) * HD;
    bf16x8 qf[HD / 32];
#pragma unroll
    for (int c = 0; c < HD / 32; ++c) {
        const u32x4 v = rvalid ? *reinterpret_cast<const u32x4*>(q + qrow + 8 * g4 + 32 * c) : u32x4{0u, 0u, 0u, 0u};
        qf[c] = __builtin_bit_cast(bf16x8, v);
    }
    const float scale_log2 = scale * 1.44269504088896340736f;
    float m_i = -INFINITY, l_i = 0.f;
    f32x4 o[HD / 16];
#pragma unroll
    for (int j = 0; j < HD / 16; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // every thread stages KCH 16-byte K chunks and one V item (4 keys x 8
    // dims, transposed in registers into 8 dim rows of 4 keys); the next
    // tile's loads are in flight while the current tile is computed
    u32x4 kreg[KCH], vreg[4];
    const int vk4 = tid / CH, vch = tid - (tid / CH) * CH;  // V item: key group of 4, dim chunk
    const bool vload = tid < VIT;
    int kt_fetch = k0;
#define MD_FETCH_TILE(kt0_)                                                                                   \
    {                                                                                                         \
        _Pragma("unroll") for (int j = 0; j < KCH; ++j) {                                                     \
            const int i = tid + BLOCK * j;                                                                    \
            const int kk = i / CH, ch = i - (i / CH) * CH;                                                    \
            const int key = (kt0_) + kk;                                                                      \
            kreg[j] = key < k1 ? *reinterpret_cast<const u32x4*>(Kc + (kvbase + key) * HD + ch * 8)           \
                               : u32x4{0u, 0u, 0u, 0u};                                                       \
        }                                                                                                     \
        _Pragma("unroll") for (int e = 0; e < 4; ++e) {                                                       \
            const int key = (kt0_) + vk4 * 4 + e;                                                             \
            vreg[e] = (vload && key < k1) ? *reinterpret_cast<const u32x4*>(Vc + (kvbase + key) * HD + vch * 8) \
                                          : u32x4{0u, 0u, 0u, 0u};                                            \
        }                                                                                                     \
    }
    if (k0 < k1) MD_FETCH_TILE(kt_fetch);
    for (int kt0 = k0; kt0 < k1; kt0 += MKT) {
        __syncthreads();
#pragma unroll
        for (int j = 0; j < KCH; ++j) {
            const int i = tid + BLOCK * j;
            const int kk = i / CH, ch = i - (i / CH) * CH;
            *reinterpret_cast<u32x4*>(&Ks[kk][ch * 8]) = kreg[j];
        }
        if (vload) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // word j of each key holds dims 2j (low half) and 2j+1 (high half)
                const uint32_t a0 = vreg[0][j], a1 = vreg[1][j], a2 = vreg[2][j], a3 = vreg[3][j];
                *reinterpret_cast<u32x2*>(&Vt[vch * 8 + 2 * j][vk4 * 4]) =
                    u32x2{(a0 & 0xffffu) | (a1 << 16), (a2 & 0xffffu) | (a3 << 16)};
                *reinterpret_cast<u32x2*>(&Vt[vch * 8 + 2 * j + 1][vk4 * 4]) =
                    u32x2{(a0 >> 16) | (a1 & 0xffff0000u), (a2 >> 16) | (a3 & 0xffff0000u)};
            }
        }
        __syncthreads();
        if (kt0 + MKT < k1) MD_FETCH_TILE(kt0 + MKT);

        // S^T for four 16-key blocks: st[kb][i] = S[row][kt0 + 16 kb + 4 g4 + i]
        f32x4 st[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            st[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < HD / 32; ++c) {
                const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&Ks[kb * 16 + c16][8 * g4 + 32 * c]));
                st[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[c], st[kb], 0, 0, 0);
            }
        }
        // scores in the log2 domain: s = scale * log2(e) * q.k, so that
        // e^{scale q.k - m} = 2^{s - m'} with the native exp2
        float p[4][4];
        float tmax = -INFINITY;
        if (kt0 + MKT <= k1 && kt0 + MKT <= L) {
            // the whole tile lies in the cached prefix: every key is visible
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p[kb][i] = st[kb][i] * scale_log2;
                    tmax = fmaxf(tmax, p[kb][i]);
                }
        } else {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int kidx = kt0 + kb * 16 + 4 * g4 + i;
                    bool vis = kidx < k1;
                    if (vis && kidx >= L) vis = (anc >> (kidx - L)) & 1ull;
                    p[kb][i] = vis ? st[kb][i] * scale_log2 : -INFINITY;
                    tmax = fmaxf(tmax, p[kb][i]);
                }
            }
        }
        tmax = fmaxf(tmax, xor16(tmax));
        tmax = fmaxf(tmax, xor32(tmax));
        const float m_new = fmaxf(m_i, tmax);
        const float mref = m_new == -INFINITY ? 0.f : m_new;  // rows with no visible key yet
        const float alpha = __builtin_amdgcn_exp2f(m_i - mref);
        float psum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[kb][i] = __builtin_amdgcn_exp2f(p[kb][i] - mref);
                psum += p[kb][i];
            }
        psum += xor16(psum);
        psum += xor32(psum);
        l_i = l_i * alpha + psum;
        // the running max of most rows stops moving after the first tiles
        if (__ballot(m_new != m_i)) {
#pragma unroll
            for (int j = 0; j < HD / 16; ++j) o[j] *= alpha;
        }
        m_i = m_new;

        // O^T += V^T P^T over two 32-key halves
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int kb0 = 2 * half, kb1 = 2 * half + 1;
            const bf16x8 pb = {(__bf16)p[kb0][0], (__bf16)p[kb0][1], (__bf16)p[kb0][2], (__bf16)p[kb0][3],
                               (__bf16)p[kb1][0], (__bf16)p[kb1][1], (__bf16)p[kb1][2], (__bf16)p[kb1][3]};
#pragma unroll
            for (int j = 0; j < HD / 16; ++j) {
                const u32x2 lo = *reinterpret_cast<const u32x2*>(&Vt[16 * j + c16][kb0 * 16 + 4 * g4]);
                const u32x2 hi = *reinterpret_cast<const u32x2*>(&Vt[16 * j + c16][kb1 * 16 + 4 * g4]);
                const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
                o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, o[j], 0, 0, 0);
            }
        }
    }
#undef MD_FETCH_TILE

    if (rvalid) {
        const int64_t row = ((int64_t)b * N + node) * Hq + h;
#pragma unroll
        for (int j = 0; j < HD / 16; ++j)
            *reinterpret_cast<f32x4*>(po + (row * splits + s) * HD + 16 * j + 4 * g4) = o[j];
        if (g4 == 0) {
            pm[row * splits + s] = m_i;
            pl[row * splits + s] = l_i;
        }
    }
}

// out = sum_s 2^{m_s - M} o_s / sum_s 2^{m_s - M} l_s  (M = max_s m_s; the row
// statistics are kept in the log2 domain)
template <typename T>
__global__ void k_attn_combine(int hd, int splits, const float* __restrict__ po, const float* __restrict__ pm,
                               const float* __restrict__ pl, T* __restrict__ out) {
    const int64_t row = blockIdx.x;
    const int c = threadIdx.x;
    float M = -INFINITY;
#pragma unroll 8
    for (int s = 0; s < splits; ++s) M = fmaxf(M, pm[row * splits + s]);
    float num = 0.f, den = 0.f;
#pragma unroll 8
    for (int s = 0; s < splits; ++s) {
        const float ms = pm[row * splits + s];
        const float wgt = ms == -INFINITY ? 0.f : exp2f(ms - M);
        num = fmaf(wgt, po[(row * splits + s) * hd + c], num);
        den = fmaf(wgt, pl[row * splits + s], den);
    }
    st(out, row * hd + c, num / den);
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

template <typename T>
hipError_t launch_typed(const DevTree& t, int B, int Hq, int Hkv, int hd, int Lcap, int max_len, const void* q,
                        const void* Kc, const void* Vc, const int32_t* lens, float scale, void* out, void* ws,
                        hipStream_t st_) {
    const AttnPlan p = attention_plan(sizeof(T) == 2, B, t.n, Hq, Hkv, hd, max_len);
    const int64_t R = (int64_t)B * t.n * Hq;
    char* w = reinterpret_cast<char*>(ws);
    float* po = reinterpret_cast<float*>(w);
    w += align256((size_t)R * p.splits * hd * 4);
    float* pm = reinterpret_cast<float*>(w);
    w += align256((size_t)R * p.splits * 4);
    float* pl = reinterpret_cast<float*>(w);
    const dim3 grid((unsigned)(B * Hkv * p.qtiles * p.splits));
    const T* qq = reinterpret_cast<const T*>(q);
    const T* kk = reinterpret_cast<const T*>(Kc);
    const T* vv = reinterpret_cast<const T*>(Vc);
    if constexpr (sizeof(T) == 2) {
        const int ngroups = B * Hkv * p.splits;
        const dim3 mgrid((unsigned)(8 * p.qtiles * ((ngroups + 7) / 8)));
        if (hd == 64)
            hipLaunchKernelGGL(k_attn_mfma<64>, mgrid, dim3(BLOCK), 0, st_, t, Hq, Hkv, Lcap, max_len, qq, kk, vv,
                               lens, scale, p.splits, p.chunk, p.qtiles, ngroups, po, pm, pl);
        else
            hipLaunchKernelGGL(k_attn_mfma<128>, mgrid, dim3(BLOCK), 0, st_, t, Hq, Hkv, Lcap, max_len, qq, kk, vv,
                               lens, scale, p.splits, p.chunk, p.qtiles, ngroups, po, pm, pl);
    } else {
        if (hd == 64)
            hipLaunchKernelGGL((k_attn_fma<T, 64>), grid, dim3(BLOCK), 0, st_, t, Hq, Hkv, Lcap, max_len, qq, kk, vv,
                               lens, scale, p.splits, p.chunk, p.qtiles, po, pm, pl);
        else
            hipLaunchKernelGGL((k_attn_fma<T, 128>), grid, dim3(BLOCK), 0, st_, t, Hq, Hkv, Lcap, max_len, qq, kk, vv,
                               lens, scale, p.splits, p.chunk, p.qtiles, po, pm, pl);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_attn_combine<T>, dim3((unsigned)R), dim3(hd), 0, st_, hd, p.splits, po, pm, pl,
                       reinterpret_cast<T*>(out));
    return hipGetLastError();
}

// resident blocks per CU of the kernel that will run (one round of blocks)
int attention_occupancy(int dt, int hd) {
    int n = 0;
    hipError_t e;
    if (dt == 0)
        e = hd == 64 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_attn_fma<float, 64>, BLOCK, 0)
                     : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_attn_fma<float, 128>, BLOCK, 0);
    else
        e = hd == 64 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_attn_mfma<64>, BLOCK, 0)
                     : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_attn_mfma<128>, BLOCK, 0);
    if (e != hipSuccess || n < 1) n = 2;
    return n;
}

}  // namespace

AttnPlan attention_plan(int dt, int B, int N, int Hq, int Hkv, int hd, int max_len) {
    AttnPlan p;
    const int qt = dt == 0 ? QT : MQT;
    const int kt = dt == 0 ? KT : MKT;
    p.rows = N * (Hq / Hkv);
    p.qtiles = (p.rows + qt - 1) / qt;
    const int base = B * Hkv * p.qtiles;
    const int tiles = (max_len + N + kt - 1) / kt;
    // split the keys so that one round of resident blocks covers the grid
    const int target = device_cus() * attention_occupancy(dt, hd);
    int splits = target / base;
    if (splits > tiles) splits = tiles;
    if (splits < 1) splits = 1;
    const int tiles_per = (tiles + splits - 1) / splits;
    p.chunk = tiles_per * kt;
    p.splits = (max_len + N + p.chunk - 1) / p.chunk;
    return p;
}

size_t attention_ws_bytes(int dt, int B, int N, int Hq, int Hkv, int hd, int max_len) {
    const AttnPlan p = attention_plan(dt, B, N, Hq, Hkv, hd, max_len);
    const size_t R = (size_t)B * N * Hq;
    return align256(R * p.splits * hd * 4) + 2 * align256(R * p.splits * 4);
}

hipError_t attention_launch(const DevTree& t, int dt, int B, int Hq, int Hkv, int hd, int Lcap, int max_len,
                            const void* q, const void* Kc, const void* Vc, const int32_t* lens, float scale,
                            void* out, void* ws, hipStream_t s) {
    if (dt == 0) return launch_typed<float>(t, B, Hq, Hkv, hd, Lcap, max_len, q, Kc, Vc, lens, scale, out, ws, s);
    return launch_typed<uint16_t>(t, B, Hq, Hkv, hd, Lcap, max_len, q, Kc, Vc, lens, scale, out, ws, s);
}
