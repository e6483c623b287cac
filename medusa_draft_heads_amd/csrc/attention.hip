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
#include <math.h>

#include "md_internal.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int QT = 16;  // query rows per block
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
            sc = vis ? sc * scale : -INFINITY;
            const float mx = wave_max(sc);
            const float m_new = fmaxf(m_i[j], mx);
            const float alpha = (m_new == -INFINITY) ? 1.f : expf(m_i[j] - m_new);
            const float p = vis ? expf(sc - m_new) : 0.f;
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

// out = sum_s e^{m_s - M} o_s / sum_s e^{m_s - M} l_s  (M = max_s m_s)
template <typename T>
__global__ void k_attn_combine(int hd, int splits, const float* __restrict__ po, const float* __restrict__ pm,
                               const float* __restrict__ pl, T* __restrict__ out) {
    const int64_t row = blockIdx.x;
    const int c = threadIdx.x;
    float M = -INFINITY;
    for (int s = 0; s < splits; ++s) M = fmaxf(M, pm[row * splits + s]);
    float num = 0.f, den = 0.f;
    for (int s = 0; s < splits; ++s) {
        const float ms = pm[row * splits + s];
        const float wgt = ms == -INFINITY ? 0.f : expf(ms - M);
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
    if (hd == 64)
        hipLaunchKernelGGL((k_attn_fma<T, 64>), grid, dim3(BLOCK), 0, st_, t, Hq, Hkv, Lcap, max_len, qq, kk, vv, lens,
                           scale, p.splits, p.chunk, p.qtiles, po, pm, pl);
    else
        hipLaunchKernelGGL((k_attn_fma<T, 128>), grid, dim3(BLOCK), 0, st_, t, Hq, Hkv, Lcap, max_len, qq, kk, vv,
                           lens, scale, p.splits, p.chunk, p.qtiles, po, pm, pl);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_attn_combine<T>, dim3((unsigned)R), dim3(hd), 0, st_, hd, p.splits, po, pm, pl,
                       reinterpret_cast<T*>(out));
    return hipGetLastError();
}

}  // namespace

AttnPlan attention_plan(int dt, int B, int N, int Hq, int Hkv, int hd, int max_len) {
    (void)dt;
    (void)hd;
    AttnPlan p;
    p.rows = N * (Hq / Hkv);
    p.qtiles = (p.rows + QT - 1) / QT;
    const int base = B * Hkv * p.qtiles;
    const int tiles = (max_len + N + KT - 1) / KT;
    int splits = (1024 + base - 1) / base;
    if (splits > tiles) splits = tiles;
    if (splits < 1) splits = 1;
    const int tiles_per = (tiles + splits - 1) / splits;
    p.chunk = tiles_per * KT;
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
