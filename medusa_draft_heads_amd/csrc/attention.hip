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
// them (the bf16 path writes its output rows divided by the running sum and
// scaled by a power of two, as 16-bit floats: half the bytes, rounding 2^-11
// against the 2^-9 of the bf16 result); a combine kernel merges the key
// ranges by log-sum-exp.
//
// bf16 storage runs on the matrix cores (v_mfma_f32_16x16x32_bf16): a wave
// owns one or two groups of 16 query rows and computes, per group,
// S^T = K Q^T per 16-key block, then
// O^T += V^T P^T. In this orientation a lane keeps one query row (lane % 16)
// in both the score and the output accumulators, so the running max, the
// rescale and the bf16 P operand never leave the lane. K and V tiles of 32
// keys go from memory straight into LDS (buffer->LDS loads) in the cache's
// own row layout, chunks permuted per row against bank conflicts, three
// stages with two in flight; the V^T operand comes from gfx950's
// transposing LDS read (ds_read_b64_tr_b16), so V is never transposed by
// hand. float32 storage (small workloads) uses an LDS-tiled FMA kernel.
#include <math.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "md_internal.h"
#include "md_wave.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int QT = 16;  // query rows per block (FMA kernel)
constexpr int MQT1 = 64;  // query rows per block of the MFMA kernel per 16-row group a wave holds (4 waves)
constexpr int DKT = 32; // keys per tile (MFMA kernel)
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
// With (request, kv head) pairs a multiple of 8: every block of one pair on
// one XCD (pair p on XCD p % 8), so its K and V and its query rows are each
// fetched once into that XCD's L2, whatever the query tile and key range.
__device__ __forceinline__ void xcd_head_decode(int id, int qtiles, int splits, int& group, int& qt) {
    const int x = id & 7, u = id >> 3, per = qtiles * splits;
    const int j = u / per, rem = u - j * per;
    qt = rem / splits;
    group = (j * 8 + x) * splits + (rem - qt * splits);
}

// word 3 of a raw buffer resource on this chip family (32-bit data format, no swizzle)
constexpr int RSRC3 = 0x00020000;
typedef __attribute__((address_space(3))) void* lds_ptr;
typedef short v4i16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void dmab(__amdgpu_buffer_rsrc_t r, unsigned char* dst, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)dst, 16, off, 0, 0, 0);
}

// K and V tiles keep the cache's row layout in LDS (one key a row, HD * 2
// bytes), with the 16-byte chunks of key row k permuted: chunk c sits in
// slot c ^ swz(k). K fragments are 16 rows x one chunk (swzK spreads 16
// consecutive rows over 16 slots); V^T fragments come from the transposing
// read below, 4 rows x 2 chunks per 16 lanes (swzV spreads 8 consecutive
// rows over distinct chunk pairs).
template <int CPR>
__device__ __forceinline__ int swzK(int k) {
    return k % CPR;
}
template <int CPR>
__device__ __forceinline__ int swzV(int k) {
    return (2 * (k % 4) + 8 * ((k / 4) % 2)) % CPR;
}

// ds_read_b64_tr_b16: within each 16-lane group, lane 4r + j receives as its
// element e the 16-bit word j of the 8 bytes addressed by lane 4e + r of the
// group. So if lane a of group g addresses V[key0 + 4g + a/4][d0 + 4(a%4)],
// lane c of the group receives V[key0 + 4g + e][d0 + c], e = 0..3: four
// consecutive keys of one dimension, the layout of a V^T operand fragment.
__device__ __forceinline__ u32x2 lds_tr4(const unsigned char* p) {
    const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p));
    return __builtin_bit_cast(u32x2, v);
}

// One block: 64 RG query rows (4 waves x RG groups of 16) of one (request,
// kv head) against the keys [k0, k1) of its split, DKT keys a tile; with RG
// = 2 every K and V fragment a wave reads from LDS serves both its groups. K and V tiles go from
// memory straight into LDS (buffer->LDS loads, 16 bytes a lane, one
// instruction per 1 KB piece) in three separately named stage buffers with
// two tiles in flight, so no register staging, no transposing writes and one
// barrier per tile.
template <int HD, int RG>
__global__ __launch_bounds__(BLOCK, RG == 1 ? 3 : 2) void k_attn_mfma(DevTree t, int Hq, int Hkv, int Lcap, int max_len,
                                                     const uint16_t* __restrict__ q, const uint16_t* __restrict__ Kc,
                                                     const uint16_t* __restrict__ Vc, const int32_t* __restrict__ lens,
                                                     float scale, int splits, int chunk, int qtiles, int ngroups,
                                                     int head_map, uint16_t* __restrict__ po, float* __restrict__ pm,
                                                     float* __restrict__ pl, float* __restrict__ pe) {
    constexpr int CPR = HD / 8;          // 16-byte chunks per key row
    constexpr int ROWB = HD * 2;         // bytes per key row
    constexpr int TILEB = DKT * ROWB;    // bytes of one K (or V) tile
    constexpr int NPK = TILEB / 1024;    // 1 KB pieces per tile
    constexpr int KPP = 1024 / ROWB;     // keys per piece
    constexpr int PPW = 2 * (NPK / 4);   // pieces each wave loads per stage (K and V)
    static_assert(NPK % 4 == 0 && KPP * CPR == MD_WAVE, "whole pieces, one lane per 16-byte chunk");
    __shared__ __align__(1024) unsigned char sb0[2 * TILEB];
    __shared__ __align__(1024) unsigned char sb1[2 * TILEB];
    __shared__ __align__(1024) unsigned char sb2[2 * TILEB];

    int grp, qt;
    if (head_map)
        xcd_head_decode(blockIdx.x, qtiles, splits, grp, qt);
    else if (!xcd_group_decode(blockIdx.x, qtiles, ngroups, grp, qt))
        return;
    const int s = grp % splits;
    const int g = (grp / splits) % Hkv;
    const int b = grp / (splits * Hkv);
    const int group = Hq / Hkv;
    const int N = t.n;
    const int rows = N * group;
    const int L = min(max(lens[b], 0), max_len);
    const int nkeys = L + N;
    const int k0 = s * chunk, k1 = min(k0 + chunk, nkeys);
    const int tid = threadIdx.x, lane = tid & (MD_WAVE - 1);
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int g4 = lane >> 4, c16 = lane & 15;
    const int64_t kvbase = ((int64_t)b * Hkv + g) * Lcap;

    // this lane's query rows (the N index of both products): one in each of
    // the wave's RG groups of 16 rows, which share every K and V fragment
    static_assert(RG == 1 || RG == 2, "one or two 16-row groups a wave");
    constexpr int MQT = MQT1 * RG;  // query rows per block
    bool rvalid[RG];
    int node[RG], hq[RG];
    uint64_t anc[RG];
    bf16x8 qf[RG][HD / 32];
#pragma unroll
    for (int gi = 0; gi < RG; ++gi) {
        const int r = qt * MQT + (w * RG + gi) * 16 + c16;
        rvalid[gi] = r < rows;
        node[gi] = rvalid[gi] ? r / group : 0;
        hq[gi] = g * group + (rvalid[gi] ? r - (r / group) * group : 0);
        anc[gi] = rvalid[gi] ? t.anc[node[gi]] : 0ull;
        const int64_t qrow = (((int64_t)b * N + node[gi]) * Hq + hq[gi]) * HD;
#pragma unroll
        for (int c = 0; c < HD / 32; ++c) {
            const u32x4 v =
                rvalid[gi] ? *reinterpret_cast<const u32x4*>(q + qrow + 8 * g4 + 32 * c) : u32x4{0u, 0u, 0u, 0u};
            qf[gi][c] = __builtin_bit_cast(bf16x8, v);
        }
    }
    const float scale_log2 = scale * 1.44269504088896340736f;
    float m_i[RG], l_i[RG];
    f32x4 o[RG][HD / 16];
#pragma unroll
    for (int gi = 0; gi < RG; ++gi) {
        m_i[gi] = -INFINITY;
        l_i[gi] = 0.f;
#pragma unroll
        for (int j = 0; j < HD / 16; ++j) o[gi][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // keys past nkeys read as zero (and are masked); the cache rows of this
    // (request, kv head) bound every load
    const __amdgpu_buffer_rsrc_t rK =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Kc + kvbase * HD), 0, nkeys * ROWB, RSRC3);
    const __amdgpu_buffer_rsrc_t rV =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Vc + kvbase * HD), 0, nkeys * ROWB, RSRC3);
    // piece p of a tile holds keys KPP p .. KPP p + KPP - 1; the lane writes
    // slot lane % CPR of key KPP p + lane / CPR and loads the chunk that
    // belongs there
    const int lkey = lane / CPR, lslot = lane % CPR;
    auto issue = [&](int kt0, unsigned char* stg) {
#pragma unroll
        for (int jj = 0; jj < NPK / 4; ++jj) {
            const int p = w + 4 * jj, key = KPP * p + lkey;
            dmab(rK, stg + p * 1024, (uint32_t)(kt0 + key) * ROWB + 16 * (lslot ^ swzK<CPR>(key)));
        }
#pragma unroll
        for (int jj = 0; jj < NPK / 4; ++jj) {
            const int p = w + 4 * jj, key = KPP * p + lkey;
            dmab(rV, stg + TILEB + p * 1024, (uint32_t)(kt0 + key) * ROWB + 16 * (lslot ^ swzV<CPR>(key)));
        }
    };

    auto compute = [&](int kt0, const unsigned char* sK) {
        const unsigned char* sV = sK + TILEB;
        // S^T for two 16-key blocks: st[gi][kb][i] = S[row of group gi][kt0 + 16 kb + 4 g4 + i]
        f32x4 st[RG][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int gi = 0; gi < RG; ++gi) st[gi][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int key = 16 * kb + c16;
#pragma unroll
            for (int c = 0; c < HD / 32; ++c) {
                const bf16x8 a = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(sK + key * ROWB + 16 * ((g4 + 4 * c) ^ swzK<CPR>(key))));
#pragma unroll
                for (int gi = 0; gi < RG; ++gi)
                    st[gi][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[gi][c], st[gi][kb], 0, 0, 0);
            }
        }
        // scores in the log2 domain: s = scale * log2(e) * q.k, so that
        // e^{scale q.k - m} = 2^{s - m'} with the native exp2
        const bool in_prefix = kt0 + DKT <= k1 && kt0 + DKT <= L;  // every key of the tile is visible
        bf16x8 pb[RG];
#pragma unroll
        for (int gi = 0; gi < RG; ++gi) {
            float p[2][4];
            float tmax = -INFINITY;
            if (in_prefix) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        p[kb][i] = st[gi][kb][i] * scale_log2;
                        tmax = fmaxf(tmax, p[kb][i]);
                    }
            } else {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int kidx = kt0 + kb * 16 + 4 * g4 + i;
                        bool vis = kidx < k1;
                        if (vis && kidx >= L) vis = (anc[gi] >> (kidx - L)) & 1ull;
                        p[kb][i] = vis ? st[gi][kb][i] * scale_log2 : -INFINITY;
                        tmax = fmaxf(tmax, p[kb][i]);
                    }
                }
            }
            // Lazy reference: P = 2^(s - m_i) with m_i the row's reference,
            // moved only when a score passes it by more than 8 (P stays below
            // 2^8); the four lanes of a row always share m_i. l_i sums this
            // lane's keys only (one reduction at the end).
            if (__ballot(tmax > m_i[gi] + 8.f)) {
                tmax = fmaxf(tmax, xor16(tmax));
                tmax = fmaxf(tmax, xor32(tmax));
                if (tmax > m_i[gi]) {  // the same for the row's four lanes
                    const float alpha = __builtin_amdgcn_exp2f(m_i[gi] - tmax);  // 0 while m_i is -inf
                    l_i[gi] *= alpha;
#pragma unroll
                    for (int j = 0; j < HD / 16; ++j) o[gi][j] *= alpha;
                    m_i[gi] = tmax;
                }
            }
            const float mref = m_i[gi] == -INFINITY ? 0.f : m_i[gi];  // rows with no visible key yet
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p[kb][i] = __builtin_amdgcn_exp2f(p[kb][i] - mref);
                    l_i[gi] += p[kb][i];
                }
            // P^T operand: k index 8 g4 + e is key 4 g4 + e (e < 4) or 16 +
            // 4 g4 + e - 4 (e >= 4), as in the V^T operand below
            pb[gi] = bf16x8{(__bf16)p[0][0], (__bf16)p[0][1], (__bf16)p[0][2], (__bf16)p[0][3],
                            (__bf16)p[1][0], (__bf16)p[1][1], (__bf16)p[1][2], (__bf16)p[1][3]};
        }

        // O^T += V^T P^T over the tile's 32 keys, each V^T fragment shared by the groups
        const int vk = 4 * g4 + (c16 >> 2);  // the key this lane addresses (first 16-key block)
        const int vq = c16 & 3;
#pragma unroll
        for (int j = 0; j < HD / 16; ++j) {
            const int ch = 2 * j + (vq >> 1), bo = 8 * (vq & 1);
            const u32x2 lo = lds_tr4(sV + vk * ROWB + 16 * (ch ^ swzV<CPR>(vk)) + bo);
            const u32x2 hi = lds_tr4(sV + (vk + 16) * ROWB + 16 * (ch ^ swzV<CPR>(vk + 16)) + bo);
            const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
#pragma unroll
            for (int gi = 0; gi < RG; ++gi)
                o[gi][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[gi], o[gi][j], 0, 0, 0);
        }
    };

    // Tile i lives in buffer i % 3; two tiles are always in flight (past the
    // last one the loads repeat it, keeping the count uniform), so the wait
    // before a tile leaves one tile's loads, PPW per wave, open. The barrier
    // is LDS-only: each wave's own wait makes its pieces land, lgkmcnt(0)
    // retires its reads of the buffer the next loads overwrite.
    const int ntile = k1 > k0 ? (k1 - k0 + DKT - 1) / DKT : 0;
    auto tile_at = [&](int i) { return k0 + min(i, max(ntile - 1, 0)) * DKT; };
    auto step = [&](int i, const unsigned char* cur, unsigned char* nxt) {
        __builtin_amdgcn_s_waitcnt(md_wave::waitcnt_vm(PPW));  // PPW: the loads issue() makes per wave
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        issue(tile_at(i + 2), nxt);
        __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of this tile's work
        compute(k0 + i * DKT, cur);
    };
    if (ntile > 0) {
        issue(tile_at(0), sb0);
        issue(tile_at(1), sb1);
        int i = 0;
        for (; i + 3 <= ntile; i += 3) {
            step(i, sb0, sb2);
            step(i + 1, sb1, sb0);
            step(i + 2, sb2, sb1);
        }
        if (i < ntile) step(i, sb0, sb2);
        if (i + 1 < ntile) step(i + 1, sb1, sb0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the repeated loads land before the block ends
    }

#pragma unroll
    for (int gi = 0; gi < RG; ++gi) {
        float li = l_i[gi];
        li += xor16(li);  // the row's sum over its four lanes
        li += xor32(li);
        // the key range's output row normalised (o / l, bounded by max |V|) and
        // scaled by a power of two 2^-ex that puts its largest entry in
        // [2^14, 2^15), stored as 16-bit floats: half the bytes of the split's
        // partial rows, no overflow past the 16-bit range whatever the size of
        // V, and the full 11-bit precision for every entry within 2^-28 of the
        // row's largest. 2^ex travels beside the row.
        const float inv = li > 0.f ? 1.f / li : 0.f;
        float amax = 0.f;
#pragma unroll
        for (int j = 0; j < HD / 16; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fabsf(o[gi][j][e] * inv));
        amax = fmaxf(amax, xor16(amax));
        amax = fmaxf(amax, xor32(amax));
        // floor(log2 amax) from the exponent field (0 for zero and subnormal rows)
        const int ebits = (int)((__float_as_uint(amax) >> 23) & 0xffu);
        const int ex = ebits == 0 ? 0 : min(max(ebits - 127 - 14, -126), 127);
        const float sc = inv * __uint_as_float((uint32_t)(127 - ex) << 23 & 0x7f800000u);
        if (rvalid[gi]) {
            const int64_t row = ((int64_t)b * N + node[gi]) * Hq + hq[gi];
#pragma unroll
            for (int j = 0; j < HD / 16; ++j) {
                const f32x4 v = o[gi][j] * sc;
                const uint32_t w0 = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[0]) |
                                    ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[1]) << 16);
                const uint32_t w1 = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[2]) |
                                    ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[3]) << 16);
                *reinterpret_cast<u32x2*>(po + (row * splits + s) * HD + 16 * j + 4 * g4) = u32x2{w0, w1};
            }
            if (g4 == 0) {
                pm[row * splits + s] = m_i[gi];
                pl[row * splits + s] = li;
                pe[row * splits + s] = ldexpf(1.f, ex);
            }
        }
    }
}

// out = sum_s 2^{m_s - M} o_s / sum_s 2^{m_s - M} l_s  (M = max_s m_s; the row
// statistics are kept in the log2 domain). float32 rows (the FMA kernel's): o_s
// as accumulated, one block per query row.
__global__ void k_attn_combine(int hd, int splits, const float* __restrict__ po, const float* __restrict__ pm,
                               const float* __restrict__ pl, float* __restrict__ out) {
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
    out[row * hd + c] = num / den;
}

// The matrix-core kernel's rows: o_s / (l_s 2^{e_s}) as 16-bit floats, 2^{e_s}
// in pe. A thread owns 8 consecutive dimensions (one 16-byte load per range)
// of one row, HD / 8 threads a row, 256 / (HD / 8) rows a block; the ranges'
// rows and statistics are loaded 8 ranges at a time before they are merged
// with a running maximum (out = num / den as above, reached by rescaling
// num and den whenever the maximum rises).
template <int HD>
__global__ __launch_bounds__(256) void k_attn_combine16(int64_t R, int splits, const uint16_t* __restrict__ po,
                                                        const float* __restrict__ pm, const float* __restrict__ pl,
                                                        const float* __restrict__ pe, uint16_t* __restrict__ out) {
    constexpr int CPR = HD / 8, RPB = 256 / CPR;
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / CPR;
    const int c = threadIdx.x % CPR;
    if (row >= R) return;
    const int64_t sb = row * splits;
    float M = -INFINITY, den = 0.f;
    float num[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) num[e] = 0.f;
    for (int s0 = 0; s0 < splits; s0 += 8) {
        float ms[8], ls[8], es[8];
        u32x4 ov[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const bool ok = s0 + j < splits;
            const int64_t i = sb + (ok ? s0 + j : 0);
            ms[j] = ok ? pm[i] : -INFINITY;
            ls[j] = ok ? pl[i] : 0.f;
            es[j] = ok ? pe[i] : 0.f;
            ov[j] = ok ? *reinterpret_cast<const u32x4*>(po + i * HD + 8 * c) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (ms[j] == -INFINITY) continue;  // a range with no visible key adds nothing
            if (ms[j] > M) {
                const float a = M == -INFINITY ? 0.f : exp2f(M - ms[j]);
                den *= a;
#pragma unroll
                for (int e = 0; e < 8; ++e) num[e] *= a;
                M = ms[j];
            }
            const float wl = exp2f(ms[j] - M) * ls[j];
            den += wl;
            const float f = wl * es[j];
            const uint32_t wd[4] = {ov[j].x, ov[j].y, ov[j].z, ov[j].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint16_t hbits = (uint16_t)(wd[e >> 1] >> (16 * (e & 1)));
                num[e] = fmaf(f, (float)__builtin_bit_cast(_Float16, hbits), num[e]);
            }
        }
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    uint32_t wo[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        uint32_t u0 = __float_as_uint(num[2 * h] * inv), u1 = __float_as_uint(num[2 * h + 1] * inv);
        u0 += 0x7FFFu + ((u0 >> 16) & 1u);  // round to nearest even bf16
        u1 += 0x7FFFu + ((u1 >> 16) & 1u);
        wo[h] = (u0 >> 16) | (u1 & 0xffff0000u);
    }
    *reinterpret_cast<u32x4*>(out + row * HD + 8 * c) = u32x4{wo[0], wo[1], wo[2], wo[3]};
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

template <typename T>
hipError_t launch_typed(const DevTree& t, int B, int Hq, int Hkv, int hd, int Lcap, int max_len, const void* q,
                        const void* Kc, const void* Vc, const int32_t* lens, float scale, void* out, void* ws,
                        hipStream_t st_) {
    const AttnPlan p = attention_plan(sizeof(T) == 2, B, t.n, Hq, Hkv, hd, max_len);
    const int64_t R = (int64_t)B * t.n * Hq;
    // partial output rows: float32 as accumulated, or (matrix-core path)
    // normalised 16-bit floats
    constexpr bool kHalfRows = sizeof(T) == 2;
    typedef typename std::conditional<kHalfRows, uint16_t, float>::type P;
    char* w = reinterpret_cast<char*>(ws);
    P* po = reinterpret_cast<P*>(w);
    w += align256((size_t)R * p.splits * hd * sizeof(P));
    float* pm = reinterpret_cast<float*>(w);
    w += align256((size_t)R * p.splits * 4);
    float* pl = reinterpret_cast<float*>(w);
    w += align256((size_t)R * p.splits * 4);
    float* pe = kHalfRows ? reinterpret_cast<float*>(w) : nullptr;  // the 16-bit rows' power-of-two scales
    const dim3 grid((unsigned)(B * Hkv * p.qtiles * p.splits));
    const T* qq = reinterpret_cast<const T*>(q);
    const T* kk = reinterpret_cast<const T*>(Kc);
    const T* vv = reinterpret_cast<const T*>(Vc);
    if constexpr (sizeof(T) == 2) {
        const int ngroups = B * Hkv * p.splits;
        const int head_map = (B * Hkv) % 8 == 0;  // every (request, kv head) pair's blocks on one XCD
        const dim3 mgrid((unsigned)(head_map ? B * Hkv * p.qtiles * p.splits : 8 * p.qtiles * ((ngroups + 7) / 8)));
#define MD_ATTN(HDV, RGV)                                                                                  \
    hipLaunchKernelGGL((k_attn_mfma<HDV, RGV>), mgrid, dim3(BLOCK), 0, st_, t, Hq, Hkv, Lcap, max_len, qq, kk, vv, lens, \
                       scale, p.splits, p.chunk, p.qtiles, ngroups, head_map, po, pm, pl, pe)
        if (hd == 64 && p.rg == 2)
            MD_ATTN(64, 2);
        else if (hd == 64)
            MD_ATTN(64, 1);
        else if (p.rg == 2)
            MD_ATTN(128, 2);
        else
            MD_ATTN(128, 1);
#undef MD_ATTN
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
    if constexpr (kHalfRows) {
        const int64_t rpb = 256 / (hd / 8);
        const dim3 cgrid((unsigned)((R + rpb - 1) / rpb));
        if (hd == 64)
            hipLaunchKernelGGL(k_attn_combine16<64>, cgrid, dim3(256), 0, st_, R, p.splits, po, pm, pl, pe,
                               reinterpret_cast<uint16_t*>(out));
        else
            hipLaunchKernelGGL(k_attn_combine16<128>, cgrid, dim3(256), 0, st_, R, p.splits, po, pm, pl, pe,
                               reinterpret_cast<uint16_t*>(out));
    } else {
        hipLaunchKernelGGL(k_attn_combine, dim3((unsigned)R), dim3(hd), 0, st_, hd, p.splits, po, pm, pl,
                           reinterpret_cast<float*>(out));
    }
    return hipGetLastError();
}

// resident blocks per CU of the kernel that will run (one round of blocks)
int attention_occupancy(int dt, int hd, int rg) {
    int n = 0;
    hipError_t e;
    if (dt == 0)
        e = hd == 64 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_attn_fma<float, 64>, BLOCK, 0)
                     : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_attn_fma<float, 128>, BLOCK, 0);
    else if (rg == 2)
        e = hd == 64 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_attn_mfma<64, 2>, BLOCK, 0)
                     : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_attn_mfma<128, 2>, BLOCK, 0);
    else
        e = hd == 64 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_attn_mfma<64, 1>, BLOCK, 0)
                     : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_attn_mfma<128, 1>, BLOCK, 0);
    if (e != hipSuccess || n < 1) n = 2;
    return n;
}

}  // namespace

AttnPlan attention_plan(int dt, int B, int N, int Hq, int Hkv, int hd, int max_len) {
    AttnPlan p;
    p.rows = N * (Hq / Hkv);
    // Two 16-row query groups a wave (each K and V fragment read from LDS
    // serves both) once there are at least 128 query tiles of 64 rows: at
    // batch 4 (Hydra, L = 8,192) attention + combine 59.5 -> 53.0 us, at
    // batch 8 98.7 -> 89.8 us; at batch 1 (70B shape, 64 tiles) the fewer,
    // longer blocks gain nothing and the extra key ranges cost the combine
    // (28.0 -> 30.3 us), so one group there.
    p.rg = dt == 0 ? 1 : (B * Hkv * ((p.rows + MQT1 - 1) / MQT1) >= 128 ? 2 : 1);
    const int qt = dt == 0 ? QT : MQT1 * p.rg;
    const int kt = dt == 0 ? KT : DKT;
    p.qtiles = (p.rows + qt - 1) / qt;
    const int base = B * Hkv * p.qtiles;
    const int tiles = (max_len + N + kt - 1) / kt;
    // split the keys so that one round of resident blocks covers the grid;
    // one-group waves at two blocks a CU, though three fit: with every CU
    // holding the same number of blocks, fewer and longer ranges cost less
    // than the third block gains (70B shape, B = 1, L = 4,096, attention +
    // combine: 12 ranges 28.9 us, 8 ranges 25.7; 8B shape 17.5 -> 14.9 by
    // the halving below; 70B at L = 2,048 20.8 -> 19.9; 10 ranges, which
    // leave half the CUs a third block, 29.9)
    const int occ = attention_occupancy(dt, hd, p.rg);
    const int target = device_cus() * (dt != 0 && p.rg == 1 ? std::min(occ, 2) : occ);
    int splits = target / base;
    // short ranges cost more in the split (partial rows written and combined)
    // than they gain in parallelism: under 8 tiles a range on average, half as
    // many (at the 70B shape, B = 1: L = 2,048 24.1 -> 21.1 us with the
    // combine, L = 4,096 with 11 tiles a range 26.0 -> 27.1 us, so kept)
    if (splits >= 2 && tiles < 8 * splits) splits /= 2;
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
    return align256(R * p.splits * hd * (dt == 0 ? 4 : 2)) + (dt == 0 ? 2 : 3) * align256(R * p.splits * 4);
}

hipError_t attention_launch(const DevTree& t, int dt, int B, int Hq, int Hkv, int hd, int Lcap, int max_len,
                            const void* q, const void* Kc, const void* Vc, const int32_t* lens, float scale,
                            void* out, void* ws, hipStream_t s) {
    if (dt == 0) return launch_typed<float>(t, B, Hq, Hkv, hd, Lcap, max_len, q, Kc, Vc, lens, scale, out, ws, s);
    return launch_typed<uint16_t>(t, B, Hq, Hkv, hd, Lcap, max_len, q, Kc, Vc, lens, scale, out, ws, s);
}

// ---- the library's own attention scratch (for callers that cannot allocate)
//
// One fixed array per GPU, in the code object's device memory: the partial
// rows and statistics of md_tree_attention_noalloc. In host code the name
// `scratch` is only a host-side stand-in for the symbol; kernels get the
// device address that hipGetSymbolAddress gives for the current device, kept
// per device after the first call there. Nothing in it needs clearing: every
// launch writes each partial row and statistic it later reads. Calls that
// overlap on one GPU share the array and race.
namespace {
static __device__ __align__(256) unsigned char scratch[kAttnScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t attention_scratch(void** ptr) {
    *ptr = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}
