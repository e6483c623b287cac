// Draft heads over many rows on the matrix cores.
//
// With one hidden state per tree node ("Medusa heads versus separate draft
// model", section "Trees": a 64-node tree at batch 8 puts 512 tokens through
// the weights, past the ridge point), the heads are two dense contractions
// per head: the residual block z = W x (d x din times din x M) and the
// vocabulary projection logits = U h' (V x d times d x M). Both run as bf16
// MFMA GEMMs (v_mfma_f32_16x16x32_bf16):
//
// * phase 1 (residual): x is exact in bf16 (h, or Hydra's [h ; E[token]]),
//   so one product per term. The epilogue forms h' = base + SiLU(z + b) in
//   float32 and also stores it split as hi = bf16(h'), lo = bf16(h' - hi).
// * phase 2 (vocabulary): h' must enter with more than bf16's 8 mantissa
//   bits (rounding it to bf16 moves logits by ~1e-3 and reorders near-equal
//   candidates); as hi + lo it enters with ~16 (relative error <= 2^-17).
//   - up to 128 rows (HBM-bound): logits = U hi + U lo, two products per
//     term, in the narrow kernel (up to 64 rows) or the register-streamed
//     one (65 to 128, one row tile so U is read once); per column (row of
//     h') the block's best k logits, filtered first by a running lower
//     bound of the k-th best; the per-block lists go through the same k-way
//     merge as the GEMV path;
//   - more rows (matrix-bound): one product, U hi, and a certificate: every
//     logit of a vocabulary tile is within E of U hi (Cauchy-Schwarz with
//     the tile's largest row norm and |lo|), so only entries whose U hi + E
//     reaches a lower bound of the k-th best are kept, then re-scored in
//     float32 from hi + lo; the top k are taken over the re-scored values
//     (details at k_vocab_mfma_cert). The bounds need tiles that have
//     finished, so shapes whose row tiles would all run in the first round
//     of blocks stay on the two-product kernel (use_certified). Logits never
//     reach memory.
//
// Residual: block tile 128 weight rows x 128 activation rows, K step 64, 4
// waves of 64 x 64 (4 x 4 MFMA tiles each), operands staged in LDS (rows
// padded against bank conflicts) from registers loaded one K step ahead,
// the contraction split when the tiles alone cannot fill the GPU; over
// many Medusa rows the vocabulary kernels' pipeline instead (256 x 128
// tiles, k_residual_wide). Vocabulary: block tile 256 vocabulary rows x 128
// (many rows) or 64 (few rows) activation rows, K step 32, operands loaded
// straight from memory into LDS in three stages with two in flight, two
// blocks per CU; from 65 to 128 rows, all activation rows in one tile with
// U streamed into registers (details at the kernels). Both operands are
// row-major along the contraction, which is exactly the MFMA operand layout
// (a lane reads 8 consecutive k of one row), so nothing is transposed; an
// optional operand-order copy of U makes every fragment of the few-row
// kernels one contiguous 1 KB load. Blocks that share a weight tile (the
// activation tiles of one weight tile) get ids spaced by 8, i.e. the same
// XCD and L2.
#include <math.h>
#include <string.h>

#include <algorithm>

#include "md_internal.h"
#include "md_wave.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int BLOCK = 256;
constexpr int TR = 128;       // weight rows per tile
constexpr int TM = 128;       // activation rows per tile
constexpr int KS = 64;        // contraction elements per step
constexpr int LP = KS + 8;    // LDS row pitch (bf16 elements)
constexpr int CH = KS / 8;    // 16-byte chunks per row and step
constexpr int NLD = TR * CH / BLOCK;  // 16-byte operand chunks per thread and step
static_assert(TR == TM, "operand loops stage A and B rows with the same index");
static_assert((TR * CH) % BLOCK == 0 && NLD >= 1, "each thread stages a whole number of chunks");
constexpr int LDS_BYTES = (TR + TM) * LP * 2;  // the residual's staged operand tiles

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ bool ranks_above(float v, int i, float w, int j) { return v > w || (v == w && i < j); }

// Float <-> int with the same order (for atomicMax on a float bound).
__device__ __forceinline__ int f2o(float f) {
    const int b = __float_as_int(f);
    return b >= 0 ? b : b ^ 0x7FFFFFFF;
}
__device__ __forceinline__ float o2f(int k) { return __int_as_float(k >= 0 ? k : k ^ 0x7FFFFFFF); }

struct KW {
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

// Hydra rows: (request, parent) -> the parent's token.
struct GemmRows {
    int kind;  // 0: activation row m is h[m]; 1: row m is [h[b] ; E[tok]] of (b, parent) = divmod(m, P)
    int P, N, V;
    int8_t parents[64];
    const uint16_t* h;
    const uint16_t* E;
    const int32_t* root_tok;
    const int32_t* tree_tok;
};

// XCD-grouped block ids: the activation tiles of one weight tile get ids
// u%8 + 8*(..) so they run on one XCD and share its L2.
__device__ __forceinline__ bool decode_tile(int id, int mtiles, int units, int& unit, int& mt) {
    const int x = id & 7, u = id >> 3;
    mt = u % mtiles;
    unit = (u / mtiles) * 8 + x;
    return unit < units;
}

// One K step of a 128 x 128 tile for this wave's 64 x 64 quadrant.
template <int NS>
__device__ __forceinline__ void tile_mma(const uint16_t (*As)[LP], const uint16_t (*Bs)[TM][LP], int wr, int wc,
                                         int g4, int c16, f32x4 (&acc)[4][4]) {
#pragma unroll
    for (int kk = 0; kk < KS / 32; ++kk) {
        bf16x8 a[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
            a[rb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&As[64 * wr + 16 * rb + c16][32 * kk + 8 * g4]));
#pragma unroll
        for (int s = 0; s < NS; ++s) {
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                const bf16x8 b = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(&Bs[s][64 * wc + 16 * cb + c16][32 * kk + 8 * g4]));
#pragma unroll
                for (int rb = 0; rb < 4; ++rb)
                    acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[rb], b, acc[rb][cb], 0, 0, 0);
            }
        }
    }
}

// h' = base + SiLU(z + b) for 4 consecutive rows r.. of head hh, activation
// row m, stored as float32 and as its hi/lo bf16 split.
// bw, hw: the 4 bias and base values (bf16 pairs; bw zero without a bias).
// Where the residual epilogue also writes hi and lo in the activation
// operand order of the narrow vocabulary kernel (hi == nullptr: not written).
// Per matrix of R rows (one head's M rows, or with one shared projection the
// heads' nh * M rows as one matrix): [tile of 64 rows][K step of 32][64
// rows][64 bytes], the 16-byte chunk c of row rr in slot c ^ ((rr / 2) % 4),
// i.e. exactly the LDS image of the kernel's activation stage, so each 1 KB
// piece (16 rows) of a stage is one contiguous load. Rows past R are never
// written; their products only reach padding columns.
struct BoOut {
    uint16_t* hi;
    uint16_t* lo;
    int shared;  // 1: the heads' rows form one [nh * M][d] matrix
    int nh;
};
constexpr int kBoTile = 64;  // rows per tile of the ordered copy (the narrow kernel's activation tile)
constexpr int kBoStep = 32;  // contraction elements per K step (its stage)
__device__ __forceinline__ int64_t bo_offset(const BoOut& bo, int M, int d, int hh, int m, int r) {
    const int hq = bo.shared ? 0 : hh, g = bo.shared ? hh * M + m : m;
    const int R = bo.shared ? bo.nh * M : M;
    const int ntile = (R + kBoTile - 1) / kBoTile, nk = d / kBoStep;
    const int mt = g / kBoTile, rr = g % kBoTile, ks = r / kBoStep, c = (r / 8) % 4;
    return ((((int64_t)hq * ntile + mt) * nk + ks) * kBoTile + rr) * kBoStep + (c ^ ((rr >> 1) & 3)) * 8 + (r % 8);
}

__device__ __forceinline__ void residual_out_w(const f32x4& z, u32x2 bw, u32x2 hw, int M, int d, int hh, int m, int r,
                                               float* __restrict__ hres, float* __restrict__ hres_out,
                                               uint16_t* __restrict__ hhi, uint16_t* __restrict__ hlo,
                                               const BoOut& bo) {
    const float bb[4] = {bf_lo(bw.x), bf_hi(bw.x), bf_lo(bw.y), bf_hi(bw.y)};
    const float base[4] = {bf_lo(hw.x), bf_hi(hw.x), bf_lo(hw.y), bf_hi(hw.y)};
    f32x4 hv;
    uint32_t hi2[2] = {0u, 0u}, lo2[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float zi = z[i] + bb[i];
        const float v = base[i] + zi / (1.f + expf(-zi));
        hv[i] = v;
        const __bf16 hb = (__bf16)v;
        const float rem = v - (float)hb;
        const __bf16 lb = (__bf16)rem;
        const uint32_t hbits = __builtin_bit_cast(uint16_t, hb), lbits = __builtin_bit_cast(uint16_t, lb);
        hi2[i >> 1] |= hbits << (16 * (i & 1));
        lo2[i >> 1] |= lbits << (16 * (i & 1));
    }
    const int64_t o = ((int64_t)hh * M + m) * d + r;
    *reinterpret_cast<f32x4*>(hres + o) = hv;
    if (hres_out) *reinterpret_cast<f32x4*>(hres_out + o) = hv;
    *reinterpret_cast<u32x2*>(hhi + o) = u32x2{hi2[0], hi2[1]};
    *reinterpret_cast<u32x2*>(hlo + o) = u32x2{lo2[0], lo2[1]};
    if (bo.hi) {  // 4 outputs r..r+3 (r % 4 == 0) lie in one 16-byte chunk
        const int64_t ob = bo_offset(bo, M, d, hh, m, r);
        *reinterpret_cast<u32x2*>(bo.hi + ob) = u32x2{hi2[0], hi2[1]};
        *reinterpret_cast<u32x2*>(bo.lo + ob) = u32x2{lo2[0], lo2[1]};
    }
}
__device__ __forceinline__ u32x2 bias_words(const uint16_t* __restrict__ bias, int head0, int hh, int d, int r) {
    return bias ? *reinterpret_cast<const u32x2*>(bias + (int64_t)(head0 + hh) * d + r) : u32x2{0u, 0u};
}
__device__ __forceinline__ void residual_out(const f32x4& z, const uint16_t* __restrict__ bias, const GemmRows& rows,
                                             int brow, int M, int d, int head0, int hh, int m, int r,
                                             float* __restrict__ hres, float* __restrict__ hres_out,
                                             uint16_t* __restrict__ hhi, uint16_t* __restrict__ hlo,
                                             const BoOut& bo) {
    const u32x2 bw = bias_words(bias, head0, hh, d, r);
    const u32x2 hw = *reinterpret_cast<const u32x2*>(rows.h + (int64_t)brow * d + r);
    residual_out_w(z, bw, hw, M, d, hh, m, r, hres, hres_out, hhi, hlo, bo);
}

// Phase 1: z = W x for rows [0, nh*d) of the heads' residual matrices and
// activation rows [0, M); epilogue h' = base + SiLU(z + b) -> hres (f32) and
// its hi/lo bf16 split. With few rows the tiles alone leave most CUs idle,
// so the contraction is split in ksplit chunks: block (tile, chunk) stores
// its partial z to zpart [ksplit][nh][M][d], and k_residual_finish adds the
// chunks in a fixed order (the result does not depend on timing).
__global__ __launch_bounds__(BLOCK, 2) void k_residual_mfma(const uint16_t* __restrict__ W,
                                                            const uint16_t* __restrict__ bias, GemmRows rows, int M,
                                                            int d, int din, int nh, int head0, int mtiles, int ksplit,
                                                            float* __restrict__ zpart,
                                                            float* __restrict__ hres, float* __restrict__ hres_out,
                                                            uint16_t* __restrict__ hhi, uint16_t* __restrict__ hlo,
                                                            int* __restrict__ bound, BoOut bo) {
    __shared__ __align__(16) unsigned char smem[LDS_BYTES];
    __shared__ int s_tok[TM];
    __shared__ int s_b[TM];
    uint16_t(*As)[LP] = reinterpret_cast<uint16_t(*)[LP]>(smem);
    uint16_t(*Bs)[TM][LP] = reinterpret_cast<uint16_t(*)[TM][LP]>(smem + TR * LP * 2);
    const int units = nh * d / TR;
    const int per_split = 8 * mtiles * ((units + 7) / 8);  // block ids of one contraction chunk
    const int kc = blockIdx.x / per_split;
    const int kspan = din / ksplit, kbeg = kc * kspan;
    int unit, mt;
    if (!decode_tile(blockIdx.x - kc * per_split, mtiles, units, unit, mt)) return;
    const int row0 = unit * TR;  // over nh*d rows (a tile never straddles heads: d % 128 == 0)
    const int hh = row0 / d, r0 = row0 - hh * d;
    const int m0 = mt * TM;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g4 = lane >> 4, c16 = lane & 15, wr = w >> 1, wc = w & 1;

    // the vocabulary kernel that follows keeps a lower bound of each (head, row)'s
    // k-th best logit here; start from -inf
    if (blockIdx.x == 0)
        for (int j = tid; j < nh * M; j += BLOCK) bound[j] = f2o(-INFINITY);
    if (tid < TM) {
        const int m = m0 + tid;
        int b = m, tok = -1;
        if (rows.kind == 1 && m < M) {
            b = m / rows.P;
            const int p = rows.parents[m - b * rows.P];
            tok = p == 0 ? rows.root_tok[b] : rows.tree_tok[(int64_t)b * rows.N + p];
            if (tok < 0 || tok >= rows.V) tok = -1;  // out-of-vocabulary token: zero embedding
        }
        s_b[tid] = b;
        s_tok[tid] = tok;
    }
    __syncthreads();

    const uint16_t* Wt = W + ((int64_t)head0 * d + row0) * din;
    u32x4 ra[NLD], rb[NLD];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
            const int i = tid + BLOCK * j;
            const int r = i / CH, c = i - (i / CH) * CH;
            ra[j] = *reinterpret_cast<const u32x4*>(Wt + (int64_t)r * din + k0 + 8 * c);
            const int m = m0 + r;
            const int kc = k0 + 8 * c;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (m < M) {
                if (rows.kind == 0) {
                    v = *reinterpret_cast<const u32x4*>(rows.h + (int64_t)m * d + kc);
                } else if (kc < d) {
                    v = *reinterpret_cast<const u32x4*>(rows.h + (int64_t)s_b[r] * d + kc);
                } else if (s_tok[r] >= 0) {
                    v = *reinterpret_cast<const u32x4*>(rows.E + (int64_t)s_tok[r] * d + (kc - d));
                }
            }
            rb[j] = v;
        }
    };
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    fetch(kbeg);
    for (int k0 = kbeg; k0 < kbeg + kspan; k0 += KS) {
        __syncthreads();
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
            const int i = tid + BLOCK * j;
            const int r = i / CH, c = i - (i / CH) * CH;
            *reinterpret_cast<u32x4*>(&As[r][8 * c]) = ra[j];
            *reinterpret_cast<u32x4*>(&Bs[0][r][8 * c]) = rb[j];
        }
        __syncthreads();
        if (k0 + KS < kbeg + kspan) fetch(k0 + KS);
        tile_mma<1>(As, Bs, wr, wc, g4, c16, acc);
    }
    if (ksplit > 1) {  // partial z of this chunk: lane holds rows 64wr + 16rb + 4g4 + i of column 64wc + 16cb + c16
#pragma unroll
        for (int rb_ = 0; rb_ < 4; ++rb_)
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                const int m = m0 + 64 * wc + 16 * cb + c16;
                if (m < M)
                    *reinterpret_cast<f32x4*>(zpart + (((int64_t)kc * nh + hh) * M + m) * d + r0 + 64 * wr + 16 * rb_ +
                                              4 * g4) = acc[rb_][cb];
            }
        return;
    }

    // epilogue: lane holds z[row = 64wr + 16rb + 4g4 + i][col = 64wc + 16cb + c16]
#pragma unroll
    for (int rb_ = 0; rb_ < 4; ++rb_) {
        const int r = r0 + 64 * wr + 16 * rb_ + 4 * g4;  // row within the head, 4 consecutive
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            const int mm = 64 * wc + 16 * cb + c16;
            const int m = m0 + mm;
            if (m >= M) continue;
            residual_out(acc[rb_][cb], bias, rows, rows.kind == 0 ? m : s_b[mm], M, d, head0, hh, m, r, hres, hres_out,
                         hhi, hlo, bo);
        }
    }
}

// Sums the ksplit partial z of each (head, row, 4 consecutive outputs) in
// chunk order and applies the residual epilogue.
__global__ __launch_bounds__(BLOCK) void k_residual_finish(const float* __restrict__ zpart, int ksplit,
                                                           const uint16_t* __restrict__ bias, GemmRows rows, int M,
                                                           int d, int nh, int head0, float* __restrict__ hres,
                                                           float* __restrict__ hres_out, uint16_t* __restrict__ hhi,
                                                           uint16_t* __restrict__ hlo, BoOut bo) {
    const int64_t q = (int64_t)blockIdx.x * BLOCK + threadIdx.x;  // index of 4 outputs over [nh][M][d]
    const int64_t total = (int64_t)nh * M * d / 4;
    if (q >= total) return;
    const int64_t e = q * 4;
    const int r = (int)(e % d);
    const int64_t hm = e / d;
    const int m = (int)(hm % M), hh = (int)(hm / M);
    const int brow = rows.kind == 0 ? m : m / rows.P;
    // the epilogue's own loads go out first, then the partials 16 at a time
    // before they are added (in chunk order): one memory round trip per 16
    // chunks instead of one each
    const u32x2 bw = bias_words(bias, head0, hh, d, r);
    const u32x2 hw = *reinterpret_cast<const u32x2*>(rows.h + (int64_t)brow * d + r);
    const int64_t cs = (int64_t)nh * M * d;
    f32x4 z = *reinterpret_cast<const f32x4*>(zpart + e);
    int c = 1;
    for (; c + 16 <= ksplit; c += 16) {
        f32x4 p[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) p[j] = *reinterpret_cast<const f32x4*>(zpart + (c + j) * cs + e);
#pragma unroll
        for (int j = 0; j < 16; ++j) z += p[j];
    }
    if (c < ksplit) {
        f32x4 p[16];
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if (c + j < ksplit) p[j] = *reinterpret_cast<const f32x4*>(zpart + (c + j) * cs + e);
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if (c + j < ksplit) z += p[j];
    }
    residual_out_w(z, bw, hw, M, d, hh, m, r, hres, hres_out, hhi, hlo, bo);
}

// Phase 2: logits = U (hi + lo) for one head's VR vocabulary rows x VM
// activation rows; epilogue: per activation row and 128-row half of the
// tile, the best k logits.
//
// Operands reach LDS by direct buffer->LDS loads (16 bytes a lane; one
// instruction fills 1 KB: 16 rows x 64 bytes), two stages deep, so the next
// stage is in flight while the matrix cores work on this one; two blocks
// share a CU, so one block's waits and epilogue overlap the other's MFMAs.
// A row's 16-byte chunk c sits in slot c ^ ((row / 2) % 4) of its 64-byte
// LDS row; with that permutation the 16 rows of an MFMA operand read meet no
// bank conflict (the counters read zero).
// Buffer resources bound each operand tile to its valid rows: loads past V
// or M are dropped by the hardware, and their products are never selected.
constexpr int VR = 256;            // vocabulary rows per tile
constexpr int VM = 128;            // activation rows per tile
constexpr int VK = 32;             // contraction elements per stage (64 bytes a row)
constexpr int ROWB = VK * 2;
constexpr int A_BYTES = VR * ROWB;         // 16 KB
constexpr int B_BYTES = VM * ROWB;         // 8 KB (hi; lo follows)
constexpr int STAGE = A_BYTES + 2 * B_BYTES;  // 32 KB
constexpr int CSTAGE = A_BYTES + B_BYTES;  // 24 KB: the certified pass's single product
constexpr int CCOLS = CSTAGE / 512;          // 48 logit columns of 128 rows per stage buffer
static_assert(3 * CCOLS >= VM && 2 * (3 * CSTAGE + 4 * (2 * VM + 4)) <= 160 * 1024, "three stages, two blocks a CU");
constexpr int NPA = A_BYTES / 4096;        // 1 KB pieces a wave loads per stage: A
constexpr int NPB = B_BYTES / 4096;        // and each of hi, lo
static_assert(2 * (2 * STAGE + 4 * VM) <= 160 * 1024, "two blocks fit the LDS of one CU");
static_assert(VM * 512 == 2 * STAGE, "a half of the logit tile fills both stage buffers");
static_assert(NPA * 4096 == A_BYTES && NPB * 4096 == B_BYTES, "each wave fills whole 1 KB pieces");

// word 3 of a raw buffer resource on this chip family (32-bit data format, no swizzle)
constexpr int RSRC3 = 0x00020000;

typedef __attribute__((address_space(3))) void* lds_ptr;

__device__ __forceinline__ void dmab(__amdgpu_buffer_rsrc_t r, unsigned char* dst, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)dst, 16, off, 0, 0, 0);
}
// Non-temporal: for loads that consume whole 128-byte lines (operand-order
// fragments). With half lines (the row-major operand shape) the other half
// would be fetched again.
__device__ __forceinline__ void dmab_nt(__amdgpu_buffer_rsrc_t r, unsigned char* dst, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)dst, 16, off, 0, 0, 2);
}

// The residual over at most 16 activation rows (Hydra's first level, a few
// Medusa rows): a block owns 16 rows of the heads' W (one MFMA row block)
// over the whole contraction, its 8 waves splitting the contraction into 8
// runs. Each wave streams its run of W and of the activation rows ([h ;
// E[parent token]] for Hydra, gathered by row) straight into a ring of RP
// register stages (16 bytes a lane per fragment: W from HBM, the activation
// rows, shared by every block, from L2), then the 8 partial sums meet in LDS
// and are added in wave order (the result does not depend on timing). No
// partial sums go through memory and no second launch finishes them
// (Hydra's 4-row level: 18.7 us against 17.6 + 4.7 for the split
// contraction and its finish). Each block reads all its activation rows
// from L2, 16 KB of them per 1 KB of W at d = 4,096, so the kernel stops
// paying beyond one column block (32 and 72 rows: 26.8 and 34.2 us against
// 23.9 and 29.2), where the split-contraction kernel runs instead. RC: 16-row
// column blocks (1). OP: W is the operand-order copy (md_operand_order of
// [heads][d][din]): each fragment one consecutive 1 KB, non-temporal loads.
constexpr int kRowsWaves = 8;  // waves of k_residual_rows
constexpr int kRowsRing = 8;   // K steps in flight per wave
// byte offset of the A fragment of rows r .. r + 15 (r % 16 == 0) of one head
// at K step ks in the operand-order copy of W [heads][d][din]
__device__ __forceinline__ uint32_t w_op_frag(int r, int ks, int din) {
    return (uint32_t)(((r / 256) * (din / 32) + ks) * 16 + (r % 256) / 16) * 1024;
}
template <int RC, bool OP>
__global__ __launch_bounds__(kRowsWaves * MD_WAVE) void k_residual_rows(
    const uint16_t* __restrict__ W, const uint16_t* __restrict__ bias, GemmRows rows, int M, int d, int din, int nh,
    int head0, float* __restrict__ hres, float* __restrict__ hres_out, uint16_t* __restrict__ hhi,
    uint16_t* __restrict__ hlo, int* __restrict__ bound, BoOut bo) {
    constexpr int RP = kRowsRing;
    __shared__ f32x4 red[kRowsWaves][RC][MD_WAVE];
    __shared__ int s_tok[16 * RC];
    __shared__ int s_b[16 * RC];
    const int row0 = blockIdx.x * 16;  // over nh * d rows (d % 16 == 0: never straddles heads)
    const int hh = row0 / d, r0 = row0 - hh * d;
    const int tid = threadIdx.x, lane = tid & (MD_WAVE - 1);
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int g4 = lane >> 4, c16 = lane & 15;
    // the vocabulary kernel that follows keeps a lower bound of each (head,
    // row)'s k-th best logit here; start from -inf
    if (blockIdx.x == 0)
        for (int j = tid; j < nh * M; j += kRowsWaves * MD_WAVE) bound[j] = f2o(-INFINITY);
    if (tid < 16 * RC) {
        const int m = tid;
        int b = m, tok = -1;
        if (rows.kind == 1 && m < M) {
            b = m / rows.P;
            const int p = rows.parents[m - b * rows.P];
            tok = p == 0 ? rows.root_tok[b] : rows.tree_tok[(int64_t)b * rows.N + p];
            if (tok < 0 || tok >= rows.V) tok = -1;  // out-of-vocabulary token: zero embedding
        }
        s_b[tid] = b;
        s_tok[tid] = tok;
    }
    __syncthreads();

    // This wave's run [kb, kb + kw) of the contraction lies wholly in h or
    // in E's half (kw divides d). A: W rows row0 + c16, chunk g4 of each K
    // step; B: activation row 16 cb + c16, chunk g4. Rows past M, and E rows
    // of out-of-vocabulary tokens, get an offset past their buffer (2^31, far
    // enough that adding a K offset cannot wrap it back): they load zeros.
    const int kw = din / kRowsWaves, kb = w * kw;
    const bool in_e = rows.kind == 1 && kb >= d;
    const int dpad = (d + 255) / 256 * 256;  // rows of a head in the operand-order copy
    const __amdgpu_buffer_rsrc_t rA =
        OP ? __builtin_amdgcn_make_buffer_rsrc((void*)(W + (int64_t)(head0 + hh) * dpad * din), 0, dpad * din * 2, RSRC3)
           : __builtin_amdgcn_make_buffer_rsrc((void*)(W + ((int64_t)head0 * d + row0) * din), 0, 16 * din * 2, RSRC3);
    const __amdgpu_buffer_rsrc_t rB = in_e ? __builtin_amdgcn_make_buffer_rsrc((void*)rows.E, 0, 0x7FFFFFF0, RSRC3)
                                           : __builtin_amdgcn_make_buffer_rsrc((void*)rows.h, 0, 0x7FFFFFF0, RSRC3);
    static_assert(kRowsWaves * 32 * kRowsRing == 2048, "the applicability rule's din % 2048");
    const uint32_t aoff = OP ? w_op_frag(r0, kb / 32, din) + lane * 16 : (uint32_t)c16 * din * 2 + (uint32_t)(kb + 8 * g4) * 2;
    constexpr uint32_t kStepA = OP ? 16 * 1024 : 64;  // bytes between a lane's A pieces of consecutive K steps
    uint32_t boff[RC];
#pragma unroll
    for (int cb = 0; cb < RC; ++cb) {
        const int m = 16 * cb + c16;
        const int src = m >= M ? -1 : (in_e ? s_tok[m] : (rows.kind == 1 ? s_b[m] : m));
        const int kk0 = in_e ? kb - d : kb;
        boff[cb] = src < 0 ? 0x80000000u : (uint32_t)src * d * 2 + (uint32_t)(kk0 + 8 * g4) * 2;
    }
    u32x4 ra[RP], rb[RP][RC];
    const int nst = kw / 32;  // K steps of the run (a multiple of RP)
    auto issue = [&](int s, int j) {
        const uint32_t ko = (uint32_t)min(s, nst - 1) * 64;
        ra[j] = __builtin_amdgcn_raw_buffer_load_b128(rA, aoff + (uint32_t)min(s, nst - 1) * kStepA, 0, OP ? 2 : 0);
#pragma unroll
        for (int cb = 0; cb < RC; ++cb)
            rb[j][cb] = __builtin_amdgcn_raw_buffer_load_b128(rB, boff[cb] + ko, 0, 0);
    };
    f32x4 acc[RC];
#pragma unroll
    for (int cb = 0; cb < RC; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < RP; ++j) issue(j, j);
    for (int s0 = 0; s0 < nst; s0 += RP) {
#pragma unroll
        for (int j = 0; j < RP; ++j) {
#pragma unroll
            for (int cb = 0; cb < RC; ++cb)
                acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ra[j]),
                                                                  __builtin_bit_cast(bf16x8, rb[j][cb]), acc[cb], 0, 0,
                                                                  0);
            issue(s0 + j + RP, j);  // past the run: repeats its last step, never used
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the repeated loads land before the wave goes on
    // lane (g4, c16) holds z rows r0 + 4 g4 + i of activation row 16 cb + c16
#pragma unroll
    for (int cb = 0; cb < RC; ++cb) red[w][cb][lane] = acc[cb];
    __syncthreads();
    // thread t: 4 consecutive outputs (row quad g, activation row m)
    if (tid < 4 * 16 * RC) {
        const int g = tid / (16 * RC), m = tid - g * (16 * RC);
        if (m < M) {
            const int cb = m / 16, l = 16 * g + (m & 15);
            f32x4 z = red[0][cb][l];
#pragma unroll
            for (int ww = 1; ww < kRowsWaves; ++ww) z += red[ww][cb][l];
            residual_out(z, bias, rows, rows.kind == 0 ? m : s_b[m], M, d, head0, hh, m, r0 + 4 * g, hres, hres_out,
                         hhi, hlo, bo);
        }
    }
}

// The residual over 17 to 77 activation rows at din = 8,192 (Hydra's levels
// past the first at d = 4,096): a block owns one 128-row tile of W and one
// eighth of the contraction (1,024 elements). It first stages its eighth of
// every activation row in LDS (gathered from h and E, 2 KB a row, one zero
// row for the padding columns), then its 8 waves each stream 16 rows of W
// through a register ring and take the activation fragments from LDS, so the
// block reads its activation chunk once (where k_residual_rows read 16 KB of
// them per 1 KB of W from L2). Blocks of one chunk run on one XCD (ids x +
// 8 u: chunk x) and share its L2. The 8 partial sums per output go to zpart
// [8][nh][M][d], added by k_residual_finish in chunk order.
constexpr int kStageKC = 1024;                 // contraction elements per chunk
constexpr int kStagePitch = kStageKC + 8;      // LDS row pitch (bf16): rows 16 bytes apart mod 256
constexpr int kStageRows = 78;                 // activation rows + the zero row
static_assert(kStageRows * kStagePitch * 2 + 2 * kStageRows * 4 <= 160 * 1024, "the chunk fits the LDS");
template <int RC, bool OP>
__global__ __launch_bounds__(kRowsWaves * MD_WAVE) void k_residual_staged(
    const uint16_t* __restrict__ W, GemmRows rows, int M, int d, int din, int nh, int head0,
    float* __restrict__ zpart, int* __restrict__ bound) {
    constexpr int RP = kRowsRing;
    __shared__ __align__(16) uint16_t xs[kStageRows * kStagePitch];
    __shared__ int s_tok[kStageRows];
    __shared__ int s_b[kStageRows];
    const int kc = blockIdx.x & 7, tile = blockIdx.x >> 3;  // contraction chunk (= XCD), 128-row tile of W
    const int row0 = tile * 128;                              // over nh * d rows (d % 128 == 0)
    const int hh = row0 / d, r0 = row0 - hh * d;
    const int tid = threadIdx.x, lane = tid & (MD_WAVE - 1);
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int g4 = lane >> 4, c16 = lane & 15;
    if (blockIdx.x == 0)
        for (int j = tid; j < nh * M; j += kRowsWaves * MD_WAVE) bound[j] = f2o(-INFINITY);
    if (tid < M) {
        const int m = tid;
        int b = m, tok = -1;
        if (rows.kind == 1) {
            b = m / rows.P;
            const int p = rows.parents[m - b * rows.P];
            tok = p == 0 ? rows.root_tok[b] : rows.tree_tok[(int64_t)b * rows.N + p];
            if (tok < 0 || tok >= rows.V) tok = -1;  // out-of-vocabulary token: zero embedding
        }
        s_b[m] = b;
        s_tok[m] = tok;
    }
    __syncthreads();
    // A: W rows row0 + 16 w + c16, chunk g4 of each K step of the block's
    // chunk; the ring's first loads go out before the activation rows are
    // staged (W does not wait for them)
    const int kb = kc * kStageKC;
    const int dpad = (d + 255) / 256 * 256;  // rows of a head in the operand-order copy
    const __amdgpu_buffer_rsrc_t rA =
        OP ? __builtin_amdgcn_make_buffer_rsrc((void*)(W + (int64_t)(head0 + hh) * dpad * din), 0, dpad * din * 2, RSRC3)
           : __builtin_amdgcn_make_buffer_rsrc((void*)(W + ((int64_t)head0 * d + row0 + 16 * w) * din), 0,
                                               16 * din * 2, RSRC3);
    const uint32_t aoff = OP ? w_op_frag(r0 + 16 * w, kb / 32, din) + lane * 16
                             : (uint32_t)c16 * din * 2 + (uint32_t)(kb + 8 * g4) * 2;
    constexpr uint32_t kStepA = OP ? 16 * 1024 : 64;  // bytes between a lane's A pieces of consecutive K steps
    u32x4 ra[RP];
    constexpr int nst = kStageKC / 32;
    static_assert(nst % RP == 0, "whole rounds of the ring");
    auto issue = [&](int s, int j) {
        ra[j] = __builtin_amdgcn_raw_buffer_load_b128(rA, aoff + (uint32_t)min(s, nst - 1) * kStepA, 0, OP ? 2 : 0);
    };
#pragma unroll
    for (int j = 0; j < RP; ++j) issue(j, j);

    // the chunk [kb, kb + 1024) of every activation row (wholly in h or in
    // E's half): a thread's pieces (at most SPT) are all loaded before any is
    // stored, one memory round trip instead of one each
    const bool in_e = rows.kind == 1 && kb >= d;
    constexpr int CPRW = kStageKC / 8;  // 16-byte pieces a row
    constexpr int SPT = (kStageRows * CPRW + kRowsWaves * MD_WAVE - 1) / (kRowsWaves * MD_WAVE);
    const int npieces = (M + 1) * CPRW;
    u32x4 xv[SPT];
#pragma unroll
    for (int q = 0; q < SPT; ++q) {
        const int i = tid + q * kRowsWaves * MD_WAVE;
        const int m = i / CPRW, c = i - m * CPRW;
        xv[q] = u32x4{0u, 0u, 0u, 0u};
        if (i < npieces && m < M) {
            const int src = in_e ? s_tok[m] : (rows.kind == 1 ? s_b[m] : m);
            if (src >= 0)
                xv[q] = *reinterpret_cast<const u32x4*>((in_e ? rows.E : rows.h) + (int64_t)src * d +
                                                        (in_e ? kb - d : kb) + 8 * c);
        }
    }
#pragma unroll
    for (int q = 0; q < SPT; ++q) {
        const int i = tid + q * kRowsWaves * MD_WAVE;
        const int m = i / CPRW, c = i - m * CPRW;
        if (i < npieces) *reinterpret_cast<u32x4*>(xs + m * kStagePitch + 8 * c) = xv[q];
    }
    __syncthreads();

    uint32_t bl[RC];  // LDS element offsets of the lane's B rows (rows past M read the zero row)
#pragma unroll
    for (int cb = 0; cb < RC; ++cb) bl[cb] = (uint32_t)min(16 * cb + c16, M) * kStagePitch + 8 * g4;
    f32x4 acc[RC];
#pragma unroll
    for (int cb = 0; cb < RC; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < nst; s0 += RP) {
#pragma unroll
        for (int j = 0; j < RP; ++j) {
            const int s = s0 + j;
#pragma unroll
            for (int cb = 0; cb < RC; ++cb) {
                const bf16x8 bv = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(xs + bl[cb] + 32 * s));
                acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ra[j]), bv, acc[cb], 0, 0,
                                                                  0);
            }
            issue(s + RP, j);  // past the chunk: repeats its last step, never used
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the repeated loads land before the wave ends
    // lane (g4, c16) holds z rows r0 + 16 w + 4 g4 + i of activation row 16 cb + c16
#pragma unroll
    for (int cb = 0; cb < RC; ++cb) {
        const int m = 16 * cb + c16;
        if (m < M)
            *reinterpret_cast<f32x4*>(zpart + (((int64_t)kc * nh + hh) * M + m) * d + r0 + 16 * w + 4 * g4) = acc[cb];
    }
}

// Operand order: a copy of a row-major [rows][d] bf16 matrix in which every
// MFMA A fragment (16 rows x 32 contraction elements, 1 KB) is contiguous in
// lane order (lane l: row l % 16, elements 8 (l / 16) .. + 7), laid out
// [tile of 256 rows][K step of 32][16-row block][64 lanes][8]; rows past the
// end are zero. One K step of a 256-row tile is then 16 KB of consecutive
// memory, where the row-major layout gives 16 runs of 64 bytes per load
// instruction (the streaming rate of that shape is ~4.8 TB/s on this part,
// of consecutive 1 KB loads ~7 TB/s). Written once, when the weights load.
constexpr int OP_TILE = 256;  // rows per tile of the operand order (the vocabulary tile)
static_assert(OP_TILE == VR, "an operand-order tile is a vocabulary tile");
__device__ __forceinline__ uint32_t op_frag(int step, int rb) { return (uint32_t)(step * (OP_TILE / 16) + rb) * 1024; }

// With one projection shared by the heads (Mh > 0) there is a single U and
// activation row m ([heads][Mh][d] read as [M][d]) belongs to head m / Mh.
// NS = 2: the activations are h' = hi + lo (two products per term); NS = 1:
// they are exact in bf16 (hlo unused), e.g. the target's own hidden states.
template <int NS>
__global__ __launch_bounds__(BLOCK, 2) void k_vocab_mfma(const uint16_t* __restrict__ U,
                                                         const uint16_t* __restrict__ hhi,
                                                         const uint16_t* __restrict__ hlo, int M, int d, int V,
                                                         int nh, int head0, int vtiles, int mtiles, int kmax,
                                                         KW kk, int Mh, float* __restrict__ part_val,
                                                         int* __restrict__ part_idx, int* __restrict__ bound) {
    __shared__ __align__(1024) unsigned char sbuf0[STAGE];
    __shared__ __align__(1024) unsigned char sbuf1[STAGE];
    __shared__ float s_bound[VM];
    const int units = nh * vtiles;
    int unit, mt;
    if (!decode_tile(blockIdx.x, mtiles, units, unit, mt)) return;
    const int hh = unit / vtiles, vt = unit - hh * vtiles;
    const int v0 = vt * VR, m0 = mt * VM;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g4 = lane >> 4, c16 = lane & 15, wr = w >> 1, wc = w & 1;
    const int64_t hbase = (int64_t)hh * M * d;

    // DMA: in 1 KB piece p = w + 4 j the lane loads row 16 p + lane / 4 =
    // r0 + 64 j, chunk (lane % 4) ^ ((row / 2) % 4), the same for every j
    const int r0 = 16 * w + (lane >> 2);
    const uint32_t voff0 = (uint32_t)r0 * d * 2 + 16 * ((lane & 3) ^ ((r0 >> 1) & 3));
    const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(U + ((int64_t)(head0 + hh) * V + v0) * d), 0, min(V - v0, VR) * d * 2, RSRC3);
    const __amdgpu_buffer_rsrc_t rH =
        __builtin_amdgcn_make_buffer_rsrc((void*)(hhi + hbase + (int64_t)m0 * d), 0, min(M - m0, VM) * d * 2, RSRC3);
    const __amdgpu_buffer_rsrc_t rL =
        __builtin_amdgcn_make_buffer_rsrc((void*)(hlo + hbase + (int64_t)m0 * d), 0, min(M - m0, VM) * d * 2, RSRC3);
    auto issue = [&](int k0, unsigned char* base) {
#pragma unroll
        for (int j = 0; j < NPA; ++j) dmab(rA, base + (w + 4 * j) * 1024, voff0 + (uint32_t)(64 * j * d + k0) * 2);
#pragma unroll
        for (int j = 0; j < NPB; ++j) {
            dmab(rH, base + A_BYTES + (w + 4 * j) * 1024, voff0 + (uint32_t)(64 * j * d + k0) * 2);
            if constexpr (NS == 2)
                dmab(rL, base + A_BYTES + B_BYTES + (w + 4 * j) * 1024, voff0 + (uint32_t)(64 * j * d + k0) * 2);
        }
    };

    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // operand rows of this lane: 16 apart, so all share the slot of row c16
    const int slot = (g4 ^ ((c16 >> 1) & 3)) * 16;
    auto compute = [&](const unsigned char* sA) {
        const unsigned char* sB = sA + A_BYTES;
        bf16x8 a[8];
#pragma unroll
        for (int rb = 0; rb < 8; ++rb)
            a[rb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(sA + (128 * wr + 16 * rb + c16) * ROWB + slot));
#pragma unroll
        for (int s = 0; s < NS; ++s) {
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                const bf16x8 b = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(sB + s * B_BYTES + (64 * wc + 16 * cb + c16) * ROWB + slot));
#pragma unroll
                for (int rb = 0; rb < 8; ++rb)
                    acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[rb], b, acc[rb][cb], 0, 0, 0);
            }
        }
    };

    // two stages, unrolled so each half of the loop names its buffer (the
    // stage count d / VK is even)
    const int nk = d / VK;
    issue(0, sbuf0);
    for (int ks = 0; ks < nk; ks += 2) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        issue((ks + 1) * VK, sbuf1);
        __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of this stage's work
        compute(sbuf0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        issue(min(ks + 2, nk - 1) * VK, sbuf0);  // the last pass reloads a stage nobody reads: no branch in the loop
        __builtin_amdgcn_sched_barrier(0);
        compute(sbuf1);
    }
    if (tid < VM)
        s_bound[tid] = m0 + tid < M ? o2f(__hip_atomic_load(bound + (int64_t)hh * M + m0 + tid, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT))
                                    : INFINITY;
    // Two passes, one per 128-row half of the tile (the waves with wr == h
    // hold it). The half's logits go to LDS: column c (row of h') takes 512
    // bytes in buffer c / 64, its 16-byte groups permuted by c % 16.
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        __syncthreads();  // operand stages, or the previous half's logits, are dead
        if (wr == h) {
#pragma unroll
            for (int rb = 0; rb < 8; ++rb)
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) {
                    const int col = 64 * wc + 16 * cb + c16;
                    *reinterpret_cast<f32x4*>((wc ? sbuf1 : sbuf0) + (col & 63) * 512 + (((4 * rb + g4) ^ (col & 15)) * 16)) =
                        acc[rb][cb];
                }
        }
        __syncthreads();
        // Per column, the best k of this half's 128 vocabulary rows.
        // Candidates below the bound of the k-th best (any list's k-th best
        // is a lower bound of the final one, so nothing of the final top-k is
        // lost) are dropped first; the rest are taken by rounds of a wave
        // argmax. Wave w owns columns w, w + 4, ...; control flow is uniform
        // across the wave.
        const int vh = v0 + 128 * h;
        const int list = 2 * vt + h;
        for (int col = w; col < VM; col += 4) {
            const int m = m0 + col;
            if (m >= M) break;  // uniform: columns past M are padding
            const int k = (Mh > 0 ? kk.at(__builtin_amdgcn_readfirstlane(min(m / Mh, 7))) : kk.at(hh));
            const float T = s_bound[col];
            const unsigned char* Sc = (col < 64 ? sbuf0 : sbuf1) + (col & 63) * 512;
            float x[2];
            int cnt = 0;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int rr = lane + 64 * q;
                x[q] = vh + rr < V ? *reinterpret_cast<const float*>(Sc + (((rr >> 2) ^ (col & 15)) * 16) + (rr & 3) * 4)
                                   : -INFINITY;
                if (x[q] < T) x[q] = -INFINITY;
                cnt += __popcll(__ballot(x[q] != -INFINITY));
            }
            const int rounds = cnt < k ? cnt : k;
            float ov = -INFINITY;
            int oi = INT_MAX;
            for (int r = 0; r < rounds; ++r) {
                float bv = x[0];
                int bi = vh + lane;
                if (ranks_above(x[1], vh + lane + 64, bv, bi)) {
                    bv = x[1];
                    bi = vh + lane + 64;
                }
                md_wave::wave_argmax(bv, bi);
                if (lane == r) {
                    ov = bv;
                    oi = bi;
                }
                if (bi == vh + lane) x[0] = -INFINITY;
                if (bi == vh + lane + 64) x[1] = -INFINITY;
            }
            if (lane < kmax) {
                const int64_t o = (((int64_t)hh * M + m) * (2 * vtiles) + list) * kmax + lane;
                part_val[o] = lane < rounds ? ov : -INFINITY;
                part_idx[o] = lane < rounds ? oi : INT_MAX;
            }
            // with k candidates taken, the k-th is a lower bound for every later
            // list; one no higher than the bound read above cannot raise it, and
            // leaving its atomic out keeps tied logits (e.g. a zero row: every
            // block's k-th equals the bound) from sending all blocks' atomics to
            // one word, which took twice the kernel's streaming time
            if (rounds == k && lane == k - 1 && ov > T) atomicMax(bound + (int64_t)hh * M + m, f2o(ov));
        }
    }
}

// Few activation rows (the target's LM head over one tree, Hydra's levels):
// the vocabulary GEMM is HBM-bound there, and with one 16 KB operand stage
// per block in flight the wide kernel's blocks wait on memory latency. This
// kernel keeps two stages in flight out of three: block tile 256 vocabulary
// rows x 64 activation rows, each wave 64 x 64 (4 x 4 MFMA tiles), stages of
// 24 KB (A 16 KB, hi 4 KB, lo 4 KB) in three separately named LDS buffers,
// two blocks per CU. Same operand layout, swizzle and bounds as the wide
// kernel; one list per (activation row, vocabulary tile).
constexpr int NM = 64;                       // activation rows per tile
constexpr int NB_BYTES = NM * ROWB;          // 4 KB (hi; lo follows)
constexpr int NSTAGE = A_BYTES + 2 * NB_BYTES;  // 24 KB
static_assert(NB_BYTES == 4096, "one 1 KB piece of each of hi, lo per wave");
static_assert(2 * (3 * NSTAGE + 4 * NM) <= 160 * 1024, "two blocks fit the LDS of one CU");
static_assert(NM * VR * 4 <= 3 * NSTAGE, "the logit tile fits the three stage buffers");
constexpr int NCOLS_PER_BUF = NSTAGE / (VR * 4);  // 24 columns of 256 logits per stage buffer
constexpr int kNarrowRows = 128;  // up to this many activation rows the two-product kernels run (narrow to 64, then direct)

// BO: the activations come from the residual epilogue's ordered copy (bo_hi,
// bo_lo; see BoOut), one contiguous 1 KB load a piece, instead of 16 rows of
// 64 bytes from hhi / hlo (half cache lines, each fetched twice).
template <int NS, bool OP, bool BO>
__global__ __launch_bounds__(BLOCK, 2) void k_vocab_mfma_narrow(const uint16_t* __restrict__ U,
                                                                const uint16_t* __restrict__ hhi,
                                                                const uint16_t* __restrict__ hlo, int M, int d, int V,
                                                                int nh, int head0, int vtiles, int mtiles, int kmax,
                                                                KW kk, int Mh, float* __restrict__ part_val,
                                                                int* __restrict__ part_idx, int* __restrict__ bound,
                                                                const uint16_t* __restrict__ bo_hi,
                                                                const uint16_t* __restrict__ bo_lo) {
    __shared__ __align__(1024) unsigned char nbuf0[NSTAGE];
    __shared__ __align__(1024) unsigned char nbuf1[NSTAGE];
    __shared__ __align__(1024) unsigned char nbuf2[NSTAGE];
    __shared__ float s_bound[NM];
    const int units = nh * vtiles;
    int unit, mt;
    if (!decode_tile(blockIdx.x, mtiles, units, unit, mt)) return;
    const int hh = unit / vtiles, vt = unit - hh * vtiles;
    const int v0 = vt * VR, m0 = mt * NM;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g4 = lane >> 4, c16 = lane & 15;
    const int64_t hbase = (int64_t)hh * M * d;

    // DMA as in the wide kernel: in 1 KB piece p = w + 4 j the lane loads row
    // r0 + 64 j of A; hi and lo are one piece each (rows r0 < 64)
    const int r0 = 16 * w + (lane >> 2);
    const uint32_t voff0 = (uint32_t)r0 * d * 2 + 16 * ((lane & 3) ^ ((r0 >> 1) & 3));
    // OP: U in operand order ([head][vtiles * VR][d], tile vt contiguous):
    // piece p of a stage is the fragment of row block p, 1 KB in place
    const __amdgpu_buffer_rsrc_t rA =
        OP ? __builtin_amdgcn_make_buffer_rsrc((void*)(U + ((int64_t)(head0 + hh) * vtiles * VR + v0) * d), 0, VR * d * 2,
                                               RSRC3)
           : __builtin_amdgcn_make_buffer_rsrc((void*)(U + ((int64_t)(head0 + hh) * V + v0) * d), 0,
                                               min(V - v0, VR) * d * 2, RSRC3);
    const __amdgpu_buffer_rsrc_t rH =
        __builtin_amdgcn_make_buffer_rsrc((void*)(hhi + hbase + (int64_t)m0 * d), 0, min(M - m0, NM) * d * 2, RSRC3);
    const __amdgpu_buffer_rsrc_t rL =
        __builtin_amdgcn_make_buffer_rsrc((void*)(hlo + hbase + (int64_t)m0 * d), 0, min(M - m0, NM) * d * 2, RSRC3);
    // ordered copy: this (head, row tile)'s K steps of 4 KB; a piece whose 16
    // rows all lie past M gets an offset past the resource (zeros, no traffic)
    static_assert(kBoTile == NM && kBoStep == VK, "the ordered copy is the narrow kernel's activation stage image");
    const int64_t bo_tile = ((int64_t)hh * mtiles + mt) * (d / VK) * NM * VK;
    const __amdgpu_buffer_rsrc_t rHo =
        __builtin_amdgcn_make_buffer_rsrc((void*)(BO ? bo_hi + bo_tile : hhi), 0, (d / VK) * NB_BYTES, RSRC3);
    const __amdgpu_buffer_rsrc_t rLo =
        __builtin_amdgcn_make_buffer_rsrc((void*)(BO ? bo_lo + bo_tile : hlo), 0, (d / VK) * NB_BYTES, RSRC3);
    const uint32_t bo_off0 = 16 * w < M - m0 ? (uint32_t)w * 1024u + lane * 16 : 0xFFFFFF00u;
    auto issue = [&](int k0, unsigned char* base) {
        if constexpr (OP) {
#pragma unroll
            for (int j = 0; j < NPA; ++j)
                dmab_nt(rA, base + (w + 4 * j) * 1024, op_frag(k0 / VK, w + 4 * j) + lane * 16);
        } else {
#pragma unroll
            for (int j = 0; j < NPA; ++j) dmab(rA, base + (w + 4 * j) * 1024, voff0 + (uint32_t)(64 * j * d + k0) * 2);
        }
        if constexpr (BO) {
            const uint32_t o = bo_off0 == 0xFFFFFF00u ? bo_off0 : bo_off0 + (uint32_t)(k0 / VK) * NB_BYTES;
            dmab(rHo, base + A_BYTES + w * 1024, o);
            if constexpr (NS == 2) dmab(rLo, base + A_BYTES + NB_BYTES + w * 1024, o);
        } else {
            dmab(rH, base + A_BYTES + w * 1024, voff0 + (uint32_t)k0 * 2);
            if constexpr (NS == 2) dmab(rL, base + A_BYTES + NB_BYTES + w * 1024, voff0 + (uint32_t)k0 * 2);
        }
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int slot = (g4 ^ ((c16 >> 1) & 3)) * 16;
    auto compute = [&](const unsigned char* sA) {
        const unsigned char* sB = sA + A_BYTES;
        bf16x8 a[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
            a[rb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                                   OP ? sA + (4 * w + rb) * 1024 + lane * 16
                                                      : sA + (64 * w + 16 * rb + c16) * ROWB + slot));
#pragma unroll
        for (int s = 0; s < NS; ++s) {
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                const bf16x8 b = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(sB + s * NB_BYTES + (16 * cb + c16) * ROWB + slot));
#pragma unroll
                for (int rb = 0; rb < 4; ++rb)
                    acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[rb], b, acc[rb][cb], 0, 0, 0);
            }
        }
    };

    // Stage s lives in buffer s % 3; two stages are always in flight (past
    // the last one the loads repeat it, keeping the count uniform), so the
    // wait before a stage leaves one stage's loads, NPA + NS per wave, open.
    const int nk = d / VK;
    // The barrier is LDS-only (no release fence): a fence would also wait for
    // the loads still in flight. Each wave's own wait makes its part of stage
    // s land before it arrives; lgkmcnt(0) retires its reads of the buffer the
    // next loads overwrite; the clobber keeps the compiler's memory operations
    // on their side of it.
    static_assert(NS == 1 || NS == 2, "one or two activation pieces per wave and stage");
    constexpr int kStageLoads = NPA + NS;  // buffer->LDS loads issue() makes per wave
    auto step = [&](int s, const unsigned char* cur, unsigned char* nxt) {
        __builtin_amdgcn_s_waitcnt(md_wave::waitcnt_vm(kStageLoads));
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        issue(min(s + 2, nk - 1) * VK, nxt);
        __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of this stage's work
        compute(cur);
    };
    issue(0, nbuf0);
    issue(min(1, nk - 1) * VK, nbuf1);
    // three whole steps per iteration (no branch inside, so the compiler's
    // wait insertion sees the same load order on every path), then the tail
    int ks = 0;
    for (; ks + 3 <= nk; ks += 3) {
        step(ks, nbuf0, nbuf2);
        step(ks + 1, nbuf1, nbuf0);
        step(ks + 2, nbuf2, nbuf1);
    }
    if (ks < nk) step(ks, nbuf0, nbuf2);
    if (ks + 1 < nk) step(ks + 1, nbuf1, nbuf0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the repeated loads land before the buffers are reused
    if (tid < NM)
        s_bound[tid] = m0 + tid < M ? o2f(__hip_atomic_load(bound + (int64_t)hh * M + m0 + tid, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT))
                                    : INFINITY;
    __syncthreads();  // operand stages are dead; the logit tile takes their LDS
    // Column c (row of h') takes 1 KB in buffer c / 24; its 16-byte groups are
    // permuted by c % 16. Lane holds rows 64 w + 16 rb + 4 g4 + i of column
    // 16 cb + c16.
    auto colp = [&](int c) -> unsigned char* {
        unsigned char* b = c < NCOLS_PER_BUF ? nbuf0 : (c < 2 * NCOLS_PER_BUF ? nbuf1 : nbuf2);
        return b + (c % NCOLS_PER_BUF) * (VR * 4);
    };
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            const int col = 16 * cb + c16;
            *reinterpret_cast<f32x4*>(colp(col) + (((16 * w + 4 * rb + g4) ^ (col & 15)) * 16)) = acc[rb][cb];
        }
    __syncthreads();
    // Per column, the block's best k of its 256 vocabulary rows, filtered by
    // the running bound as in the wide kernel. Wave w owns columns w, w + 4, ...
    for (int col = w; col < NM; col += 4) {
        const int m = m0 + col;
        if (m >= M) break;  // uniform: columns past M are padding
        const int k = (Mh > 0 ? kk.at(__builtin_amdgcn_readfirstlane(min(m / Mh, 7))) : kk.at(hh));
        const float T = s_bound[col];
        const unsigned char* Sc = colp(col);
        float x[4];
        int cnt = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int rr = lane + 64 * q;
            x[q] = v0 + rr < V ? *reinterpret_cast<const float*>(Sc + (((rr >> 2) ^ (col & 15)) * 16) + (rr & 3) * 4)
                               : -INFINITY;
            if (x[q] < T) x[q] = -INFINITY;
            cnt += __popcll(__ballot(x[q] != -INFINITY));
        }
        const int rounds = cnt < k ? cnt : k;
        float ov = -INFINITY;
        int oi = INT_MAX;
        for (int r = 0; r < rounds; ++r) {
            float bv = x[0];
            int bi = v0 + lane;
#pragma unroll
            for (int q = 1; q < 4; ++q)
                if (ranks_above(x[q], v0 + lane + 64 * q, bv, bi)) {
                    bv = x[q];
                    bi = v0 + lane + 64 * q;
                }
            md_wave::wave_argmax(bv, bi);
            if (lane == r) {
                ov = bv;
                oi = bi;
            }
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (bi == v0 + lane + 64 * q) x[q] = -INFINITY;
        }
        if (lane < kmax) {
            const int64_t o = (((int64_t)hh * M + m) * vtiles + vt) * kmax + lane;
            part_val[o] = lane < rounds ? ov : -INFINITY;
            part_idx[o] = lane < rounds ? oi : INT_MAX;
        }
        if (rounds == k && lane == k - 1 && ov > T) atomicMax(bound + (int64_t)hh * M + m, f2o(ov));
    }
}

// ---- 65 to 128 activation rows: the projection streamed into registers ----
//
// Past 64 activation rows the narrow kernel needs two row tiles, and each
// re-reads the whole projection. This kernel takes all activation rows
// (5 to 8 column blocks of 16) in one tile, so U is read once: each wave
// streams its 64 vocabulary rows of U as MFMA A fragments straight into a
// ring of P register stages (16 bytes a lane per 16-row block and K step,
// P K steps of 4 KB in flight per wave). The activation rows (hi and, with
// NS = 2, lo) form the B operand, shared by the four waves; they reach LDS
// by buffer->LDS loads issued in the same stream as the A loads, P - 1 steps
// ahead, one stage per step in P separately named buffers. Block tile: 256
// vocabulary rows (one list per activation row and tile, as in the narrow
// kernel); two blocks per CU. Both kernels read U in the MFMA operand shape
// (16 rows x 64 bytes a load), which streams at about 4.8 TB/s on this part
// against 7.1 TB/s for runs of 256 bytes a row; the products and their order
// are the same, so both give the same logits bit for bit.
// N 16-byte LDS reads at la + 1024 i (i < N), in blocks of up to four that
// each end with their own wait (the results are complete when a block ends).
__device__ __forceinline__ void lds4(u32x4& a, u32x4& b, u32x4& c, u32x4& e, uint32_t la) {
    asm volatile(
        "ds_read_b128 %0, %4\n\tds_read_b128 %1, %4 offset:1024\n\tds_read_b128 %2, %4 offset:2048\n\t"
        "ds_read_b128 %3, %4 offset:3072\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(a), "=&v"(b), "=&v"(c), "=&v"(e)
        : "v"(la)
        : "memory");
}
__device__ __forceinline__ void lds2(u32x4& a, u32x4& b, uint32_t la) {
    asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:1024\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(a), "=&v"(b)
                 : "v"(la)
                 : "memory");
}
__device__ __forceinline__ void lds1(u32x4& a, uint32_t la) {
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(a) : "v"(la) : "memory");
}
template <int N>
__device__ __forceinline__ void lds_frags(u32x4 (&f)[N], uint32_t la) {
#pragma unroll
    for (int i = 0; i + 4 <= N; i += 4) lds4(f[i], f[i + 1], f[i + 2], f[i + 3], la + 1024 * i);
    constexpr int r = N & 3, b = N - r;
    if constexpr (r >= 2) lds2(f[b], f[b + 1], la + 1024 * b);
    if constexpr (r & 1) lds1(f[N - 1], la + 1024 * (N - 1));
}

template <int NS, int CB>
struct DirectCfg {
    static constexpr int STG = NS * CB * 1024;               // LDS bytes of one B stage (16 columns x 64 B a piece)
    static constexpr int NPC = NS * CB;                       // 1 KB pieces a stage
    static constexpr int NB = (NPC + 3) / 4;                  // pieces each wave loads a stage (the last repeats)
    static constexpr int P = (NPC <= 9 && CB <= 5) ? 8 : ((NPC <= 12 && CB <= 6) ? 6 : 4);  // K steps in flight
    static constexpr int CPP = (P * STG) / 16384 < 1 ? 1 : ((P * STG) / 16384 > CB ? CB : (P * STG) / 16384);
    static constexpr int SB = STG > (16384 * CPP) / P ? STG : (16384 * CPP) / P;  // bytes of each named buffer
    static constexpr int COLS_PER_BUF = SB / 1024;             // logit columns of 256 rows per buffer
    static constexpr int WAIT = 4 + (P - 2) * (NB + 4);       // loads left open when a stage is consumed
    static_assert(SB % 1024 == 0 && WAIT <= 63, "whole 1 KB columns; the wait fits the counter");
    static_assert(COLS_PER_BUF * P >= 16 * CPP, "a pass of the logit tile fits the stage buffers");
    static_assert(2 * P * SB + 2 * 4 * 128 <= 160 * 1024, "two blocks fit the LDS of one CU");
};

template <int NS, int CB, bool OP, bool BO>
__global__ __launch_bounds__(BLOCK, 2) void k_vocab_mfma_direct(const uint16_t* __restrict__ U,
                                                                const uint16_t* __restrict__ hhi,
                                                                const uint16_t* __restrict__ hlo, int M, int d, int V,
                                                                int nh, int head0, int vtiles, int kmax, KW kk, int Mh,
                                                                float* __restrict__ part_val,
                                                                int* __restrict__ part_idx, int* __restrict__ bound,
                                                                const uint16_t* __restrict__ bo_hi,
                                                                const uint16_t* __restrict__ bo_lo) {
    typedef DirectCfg<NS, CB> C;
    constexpr int P = C::P;
    __shared__ __align__(1024) unsigned char db0[C::SB];
    __shared__ __align__(1024) unsigned char db1[C::SB];
    __shared__ __align__(1024) unsigned char db2[C::SB];
    __shared__ __align__(1024) unsigned char db3[C::SB];
    __shared__ __align__(1024) unsigned char db4[P > 4 ? C::SB : 16];
    __shared__ __align__(1024) unsigned char db5[P > 5 ? C::SB : 16];
    __shared__ __align__(1024) unsigned char db6[P > 6 ? C::SB : 16];
    __shared__ __align__(1024) unsigned char db7[P > 7 ? C::SB : 16];
    __shared__ float s_bound[CB * 16];
    auto buf = [&](int j) -> unsigned char* {
        switch (j) {
            case 0: return db0;
            case 1: return db1;
            case 2: return db2;
            case 3: return db3;
            case 4: return db4;
            case 5: return db5;
            case 6: return db6;
            default: return db7;
        }
    };
    const int hh = blockIdx.x / vtiles, vt = blockIdx.x - hh * vtiles;
    if (hh >= nh) return;
    const int v0 = vt * VR;
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int g4 = lane >> 4, c16 = lane & 15;
    const int64_t hbase = (int64_t)hh * M * d;
    const int nk = d / VK;

    // A: the lane's rows are 64 w + 16 rb + c16, its 16 bytes the chunk g4 of
    // the K step (the MFMA A layout); rows past V read as zero
    const __amdgpu_buffer_rsrc_t rA =
        OP ? __builtin_amdgcn_make_buffer_rsrc((void*)(U + ((int64_t)(head0 + hh) * vtiles * VR + v0) * d), 0, VR * d * 2,
                                               RSRC3)
           : __builtin_amdgcn_make_buffer_rsrc((void*)(U + ((int64_t)(head0 + hh) * V + v0) * d), 0,
                                               min(V - v0, VR) * d * 2, RSRC3);
    const uint32_t aoff = (uint32_t)(64 * w + c16) * d * 2 + 16 * g4;
    // B: piece p of a stage is operand p / CB (hi, lo), column block p % CB;
    // the lane loads column 16 (p % CB) + lane / 4, chunk (lane % 4) ^
    // ((column / 2) % 4) (the LDS swizzle of the other kernels)
    const __amdgpu_buffer_rsrc_t rH =
        __builtin_amdgcn_make_buffer_rsrc((void*)(hhi + hbase), 0, M * d * 2, RSRC3);
    const __amdgpu_buffer_rsrc_t rL =
        __builtin_amdgcn_make_buffer_rsrc((void*)(hlo + hbase), 0, M * d * 2, RSRC3);
    const int bc = lane >> 2;
    const uint32_t boff = (uint32_t)bc * d * 2 + 16 * ((lane & 3) ^ ((bc >> 1) & 3));
    // BO: the residual epilogue's ordered copy (see BoOut): column block cb
    // is row block cb % 4 of 64-row tile cb / 4, each K step of a tile 4 KB
    // in place; blocks whose 16 rows all lie past M load nothing
    static_assert(kBoTile == 64 && kBoStep == VK, "ordered copy tiles of four 16-row blocks");
    const int64_t bo_head = (int64_t)hh * ((M + kBoTile - 1) / kBoTile) * nk * NB_BYTES / 2;
    const uint32_t bo_size = (uint32_t)((M + kBoTile - 1) / kBoTile) * nk * NB_BYTES;
    const __amdgpu_buffer_rsrc_t rHo =
        __builtin_amdgcn_make_buffer_rsrc((void*)(BO ? bo_hi + bo_head : hhi), 0, bo_size, RSRC3);
    const __amdgpu_buffer_rsrc_t rLo =
        __builtin_amdgcn_make_buffer_rsrc((void*)(BO ? bo_lo + bo_head : hlo), 0, bo_size, RSRC3);

    u32x4 ra[P][4];
    auto issue_a = [&](int s, u32x4 (&r)[4]) {
        if constexpr (OP) {  // the wave's four fragments of a K step: 4 KB in place, non-temporal
            const uint32_t o = op_frag(min(s, nk - 1), 4 * w) + lane * 16;
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) r[rb] = __builtin_amdgcn_raw_buffer_load_b128(rA, o + rb * 1024, 0, 2);
        } else {
            const uint32_t o = aoff + (uint32_t)min(s, nk - 1) * (VK * 2);
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
                r[rb] = __builtin_amdgcn_raw_buffer_load_b128(rA, o + (uint32_t)(16 * rb) * d * 2, 0, 0);
        }
    };
    auto issue_b = [&](int s, unsigned char* dst) {
        const uint32_t ko = (uint32_t)min(s, nk - 1) * (VK * 2);
#pragma unroll
        for (int j = 0; j < C::NB; ++j) {
            const int p = min(w + 4 * j, C::NPC - 1);
            const int op = p / CB, cb = p - (p / CB) * CB;
            if constexpr (BO) {
                const uint32_t o = 16 * cb < M ? ((uint32_t)(cb / 4) * nk + (uint32_t)min(s, nk - 1)) * NB_BYTES +
                                                     (uint32_t)(cb % 4) * 1024u + lane * 16
                                               : 0xFFFFFF00u;
                dmab((NS == 2 && op) ? rLo : rHo, dst + p * 1024, o);
            } else {
                const uint32_t o = boff + (uint32_t)(16 * cb) * d * 2 + ko;
                dmab((NS == 2 && op) ? rL : rH, dst + p * 1024, o);
            }
        }
    };

    f32x4 acc[4][CB];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < CB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int slot = (g4 ^ ((c16 >> 1) & 3)) * 16;
    // The B fragments are read by inline assembly that waits for them in the
    // same block: the compiler does not see these LDS reads, so it adds no
    // waits of its own for the buffer->LDS loads still in flight into other
    // stages (the explicit wait and barrier of each step order them).
    auto compute = [&](const u32x4 (&r)[4], const unsigned char* sB) {
        u32x4 bf[C::NPC];
        const uint32_t la = (uint32_t)(uintptr_t)(sB + c16 * ROWB + slot);
        lds_frags<C::NPC>(bf, la);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
#pragma unroll
            for (int cb = 0; cb < CB; ++cb) {
                const bf16x8 b = __builtin_bit_cast(bf16x8, bf[s * CB + cb]);
#pragma unroll
                for (int rb = 0; rb < 4; ++rb)
                    acc[rb][cb] =
                        __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, r[rb]), b, acc[rb][cb], 0, 0, 0);
            }
        }
    };

    // Issue order: A(0), then per step t < 0 ... each step s issues B(s + P - 1)
    // into the buffer read at step s - 1 and, after its MFMAs, A(s + P) into
    // the ring slot it just consumed. When step s starts, everything up to
    // B(s) must have landed; issued after it are A(s + 1) and P - 2 steps of
    // (B, A): 4 + (P - 2) (NB + 4) loads.
    issue_a(0, ra[0]);
#pragma unroll
    for (int j = 1; j < P; ++j) {
        issue_b(j - 1, buf(j - 1));
        issue_a(j, ra[j]);
    }
    auto step = [&](int s, int j) {
        __builtin_amdgcn_s_waitcnt(md_wave::waitcnt_vm(C::WAIT));
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        issue_b(s + P - 1, buf((j + P - 1) % P));
        __builtin_amdgcn_sched_barrier(0);
        compute(ra[j], buf(j));
        __builtin_amdgcn_sched_barrier(0);
        issue_a(s + P, ra[j]);
    };
    // whole rounds of P steps with no branch inside (the compiler's waits for
    // the ring registers then match on every path), then the tail
    int s0 = 0;
    for (; s0 + P <= nk; s0 += P) {
#pragma unroll
        for (int j = 0; j < P; ++j) step(s0 + j, j);
    }
#pragma unroll
    for (int j = 0; j < P; ++j)
        if (s0 + j < nk) step(s0 + j, j);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the repeated loads land before the buffers are reused
    // The ring is read here: the U loads of the last steps go into slots no
    // later step reads, and dropped as unused they would leave fewer loads
    // behind each stage than the counted wait assumes.
#pragma unroll
    for (int j = 0; j < P; ++j)
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) asm volatile("" ::"v"(ra[j][rb]));
    if (tid < CB * 16)
        s_bound[tid] = tid < M ? o2f(__hip_atomic_load(bound + (int64_t)hh * M + tid, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT))
                               : INFINITY;
    // Logits tile in passes of CPP column blocks: column c of a pass takes
    // 1 KB in buffer c / COLS_PER_BUF, its 16-byte groups permuted by c % 16.
    auto colp = [&](int c) -> unsigned char* { return buf(c / C::COLS_PER_BUF) + (c % C::COLS_PER_BUF) * 1024; };
#pragma unroll
    for (int cb0 = 0; cb0 < CB; cb0 += C::CPP) {
        __syncthreads();  // operand stages, or the previous pass's logits, are dead
#pragma unroll
        for (int rb = 0; rb < 4; ++rb)
#pragma unroll
            for (int cq = 0; cq < C::CPP; ++cq) {
                if (cb0 + cq < CB) {
                    const int col = 16 * cq + c16;
                    *reinterpret_cast<f32x4*>(colp(col) + (((16 * w + 4 * rb + g4) ^ (col & 15)) * 16)) =
                        acc[rb][cb0 + cq];
                }
            }
        __syncthreads();
        const int ncol = 16 * min(C::CPP, CB - cb0);
        for (int col = w; col < ncol; col += 4) {
            const int m = 16 * cb0 + col;
            if (m >= M) break;  // uniform: columns past M are padding
            const int k = (Mh > 0 ? kk.at(__builtin_amdgcn_readfirstlane(min(m / Mh, 7))) : kk.at(hh));
            const float T = s_bound[m];
            const unsigned char* Sc = colp(col);
            float x[4];
            int cnt = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int rr = lane + 64 * q;
                x[q] = v0 + rr < V ? *reinterpret_cast<const float*>(Sc + (((rr >> 2) ^ (col & 15)) * 16) + (rr & 3) * 4)
                                   : -INFINITY;
                if (x[q] < T) x[q] = -INFINITY;
                cnt += __popcll(__ballot(x[q] != -INFINITY));
            }
            const int rounds = cnt < k ? cnt : k;
            float ov = -INFINITY;
            int oi = INT_MAX;
            for (int r = 0; r < rounds; ++r) {
                float bv = x[0];
                int bi = v0 + lane;
#pragma unroll
                for (int q = 1; q < 4; ++q)
                    if (ranks_above(x[q], v0 + lane + 64 * q, bv, bi)) {
                        bv = x[q];
                        bi = v0 + lane + 64 * q;
                    }
                md_wave::wave_argmax(bv, bi);
                if (lane == r) {
                    ov = bv;
                    oi = bi;
                }
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (bi == v0 + lane + 64 * q) x[q] = -INFINITY;
            }
            if (lane < kmax) {
                const int64_t o = (((int64_t)hh * M + m) * vtiles + vt) * kmax + lane;
                part_val[o] = lane < rounds ? ov : -INFINITY;
                part_idx[o] = lane < rounds ? oi : INT_MAX;
            }
            if (rounds == k && lane == k - 1 && ov > T) atomicMax(bound + (int64_t)hh * M + m, f2o(ov));
        }
    }
}

template <int NS, bool OP, bool BO>
hipError_t launch_direct(int cb, dim3 grid, hipStream_t s, const uint16_t* U, const uint16_t* hhi, const uint16_t* hlo,
                         int M, int d, int V, int nh, int head0, int vtiles, int kmax, KW kk, int Mh, float* pv,
                         int* pi, int* bound, const uint16_t* bo_hi = nullptr, const uint16_t* bo_lo = nullptr) {
#define MD_DIRECT(CBV)                                                                                               \
    case CBV:                                                                                                        \
        hipLaunchKernelGGL((k_vocab_mfma_direct<NS, CBV, OP, BO>), grid, dim3(BLOCK), 0, s, U, hhi, hlo, M, d, V, nh,    \
                           head0, vtiles, kmax, kk, Mh, pv, pi, bound, bo_hi, bo_lo);                                 \
        break;
    switch (cb) {
        MD_DIRECT(5)
        MD_DIRECT(6)
        MD_DIRECT(7)
        MD_DIRECT(8)
        default: return hipErrorInvalidValue;
    }
#undef MD_DIRECT
    return hipGetLastError();
}

// ---- the largest row norm of each vocabulary tile (once per weight set) ----
//
// out[mat][vt] = max over the tile's rows v of sum_j U[mat][v][j]^2 (rows past
// V count 0). The squares of bf16 values are exact in float32 and a row's sum
// carries a relative rounding error below (d / 512 + 6) 2^-24, far inside the
// 2^-10 the certified pass adds to the norm's square root. A wave per row at
// a time, 16 bytes a lane per load; the lanes' sums are added in a fixed order.
__global__ __launch_bounds__(BLOCK) void k_tile_norms(const uint16_t* __restrict__ U, int V, int d, int vtiles,
                                                      float* __restrict__ out) {
    __shared__ float s_mx[BLOCK / MD_WAVE];
    const int mat = blockIdx.x / vtiles, vt = blockIdx.x - mat * vtiles;
    const int lane = threadIdx.x & (MD_WAVE - 1), w = threadIdx.x >> 6;
    float mx = 0.f;
    for (int r = w; r < VR; r += BLOCK / MD_WAVE) {
        const int v = vt * VR + r;
        if (v >= V) break;  // uniform: rows past V
        const uint16_t* row = U + ((int64_t)mat * V + v) * d;
        float acc = 0.f;
        for (int c = 8 * lane; c < d; c += 8 * MD_WAVE) {
            const u32x4 q = *reinterpret_cast<const u32x4*>(row + c);
            const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float lo = __uint_as_float(wd[e] << 16), hi = __uint_as_float(wd[e] & 0xffff0000u);
                acc = fmaf(lo, lo, acc);
                acc = fmaf(hi, hi, acc);
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, MD_WAVE);
        mx = fmaxf(mx, acc);
    }
    if (lane == 0) s_mx[w] = mx;
    __syncthreads();
    if (threadIdx.x == 0) {
        float m = s_mx[0];
        for (int i = 1; i < BLOCK / MD_WAVE; ++i) m = fmaxf(m, s_mx[i]);
        out[blockIdx.x] = m;
    }
}

// ---- certified single-product vocabulary pass (many rows) ----
//
// With h' = hi + lo' (hi = bf16(h'), lo' the exact rest), the logit is
// l = U.hi + U.lo'. The matrix cores compute only l~ = U.hi; by
// Cauchy-Schwarz |U_v.lo'| <= |U_v| |lo'|, so with N the largest row norm of
// U in a vocabulary tile every re-scored logit r_v of that tile satisfies
//     |l~_v - r_v| <= E = N ((1 + 2^-7) |lo'| + c(d) |h'|)
// where c(d) (cert_rounding_allowance) covers float32 rounding of both the
// matrix-core sums and the re-scoring below by the standard bound for
// recursive summation, |fl(sum) - sum| <= gamma_n sum |x_i y_i| <=
// gamma_n |U_v| |x| with gamma_n = n u / (1 - n u), u = 2^-24, n the longest
// chain of roundings a product goes through: d / 32 accumulator steps plus
// up to 32 inside one MFMA for U.hi, d / 64 lane steps plus 6 butterfly
// levels for the re-scoring. The 1 + 2^-7 covers lo = bf16(lo') in the
// re-scoring and the float32 norms. A tile's k-th best l~ minus E is then a
// lower bound T of the row's k-th best logit; only entries with
// l~ + E >= T can belong to the top k. Those candidates are re-scored in
// float32 from U and h' and the top k taken over the re-scored values.
constexpr int kCertCap = 8192;  // candidates kept per (head, row); more -> exact full scan of that row
constexpr int kSlots = 64;      // per-row maxima of half-tile lower bounds (their k-th largest bounds the k-th best)

// Per (head, row): |h' - bf16(h')| and |h'| (one wave per row, fixed order).
__global__ __launch_bounds__(BLOCK) void k_row_norms(const float* __restrict__ hres, int rows, int d,
                                                     float* __restrict__ lo_norm, float* __restrict__ h_norm) {
    const int row = blockIdx.x * (BLOCK / 64) + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (row >= rows) return;
    const float* x = hres + (int64_t)row * d;
    float sl = 0.f, sh = 0.f;
    for (int c = lane * 4; c < d; c += 256) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(x + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float r = v[i] - (float)(__bf16)v[i];
            sl = fmaf(r, r, sl);
            sh = fmaf(v[i], v[i], sh);
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        sl += __shfl_xor(sl, o, 64);
        sh += __shfl_xor(sh, o, 64);
    }
    if (lane == 0) {
        lo_norm[row] = sqrtf(sl) * (1.f + 0x1p-10f);  // the sums' own rounding, rounded up
        h_norm[row] = sqrtf(sh) * (1.f + 0x1p-10f);
    }
}

__global__ void k_cert_prep(int* __restrict__ bound, int* __restrict__ slots, int* __restrict__ count, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        bound[i] = f2o(-INFINITY);
        count[i] = 0;
    }
    if (i < n * kSlots) slots[i] = f2o(-INFINITY);
}

// float32 dot of a bf16 row of U with h' = hi + lo (bf16 each; products
// exact) by one wave: each lane sums its 8-element chunks in order, then a
// butterfly.
__device__ __forceinline__ float wave_dot2(const uint16_t* __restrict__ u, const uint16_t* __restrict__ xh,
                                           const uint16_t* __restrict__ xl, int d, int lane) {
    float s = 0.f;
    auto acc = [&](const u32x4& w, const u32x4& h, const u32x4& l) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            s = fmaf(bf_lo(w[e]), bf_lo(h[e]) + bf_lo(l[e]), s);
            s = fmaf(bf_hi(w[e]), bf_hi(h[e]) + bf_hi(l[e]), s);
        }
    };
    // eight column steps' loads in flight before their products, added in the
    // same order as one step at a time (the same sum, bit for bit)
    int c = lane * 8;
    for (; c + 7 * 512 < d; c += 8 * 512) {
        u32x4 w[8], h[8], l[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            w[q] = *reinterpret_cast<const u32x4*>(u + c + q * 512);
            h[q] = *reinterpret_cast<const u32x4*>(xh + c + q * 512);
            l[q] = *reinterpret_cast<const u32x4*>(xl + c + q * 512);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) acc(w[q], h[q], l[q]);
    }
    for (; c < d; c += 512)
        acc(*reinterpret_cast<const u32x4*>(u + c), *reinterpret_cast<const u32x4*>(xh + c),
            *reinterpret_cast<const u32x4*>(xl + c));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    return s;
}

// One block per (head, row m). The candidates' lower bounds give T*, the
// k-th best of them: a lower bound of the row's k-th best logit at least as
// good as the running one. Candidates whose upper bound reaches max(T, T*)
// are re-scored in float32 and the row's top k taken over the re-scored
// values. If the candidate buffer overflowed, or more than kSurv survive,
// every vocabulary row is re-scored instead (one pass, each wave keeping its
// own k best).
constexpr int kSurv = 512;
__global__ __launch_bounds__(BLOCK) void k_rescore(const uint16_t* __restrict__ U, const uint16_t* __restrict__ hhi,
                                                   const uint16_t* __restrict__ hlo, int M, int d, int V, int nh,
                                                   int head0, int shared_u, KW kk, int kmax,
                                                   const int* __restrict__ bound, const int* __restrict__ count,
                                                   const float* __restrict__ cand_ub, const float* __restrict__ cand_lb,
                                                   const int* __restrict__ cand_idx, int32_t* __restrict__ topk_idx,
                                                   float* __restrict__ topk_val) {
    __shared__ float s_v[kSurv];  // re-scored values
    __shared__ int s_i[kSurv];    // survivors' indices
    __shared__ int s_n;
    __shared__ float wv_s[BLOCK / 64];
    __shared__ int wi_s[BLOCK / 64];
    const int hh = blockIdx.x / M, m = blockIdx.x - hh * M;
    const int row = hh * M + m;  // row of h' and of the candidate arrays
    const int k = kk.at(hh);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const uint16_t* Uh = U + (shared_u ? 0 : (int64_t)(head0 + hh) * V * d);
    const uint16_t* xh = hhi + (int64_t)row * d;
    const uint16_t* xl = hlo + (int64_t)row * d;
    const int cnt = count[row];
    // block argmax of (value, index) strictly below (pv, pi) over one value per thread
    auto block_pick1 = [&](float v, int i, float& ov, int& oi) {
        float bv = v;
        int bi = i;
        md_wave::wave_argmax(bv, bi);
        if (lane == 0) {
            wv_s[w] = bv;
            wi_s[w] = bi;
        }
        __syncthreads();
        bv = wv_s[0];
        bi = wi_s[0];
        for (int w2 = 1; w2 < BLOCK / 64; ++w2)
            if (ranks_above(wv_s[w2], wi_s[w2], bv, bi)) {
                bv = wv_s[w2];
                bi = wi_s[w2];
            }
        __syncthreads();
        ov = bv;
        oi = bi;
    };
    if (tid == 0) s_n = 0;
    __syncthreads();
    bool full = cnt > kCertCap;
    if (!full) {
        float Tf = o2f(bound[row]);
        if (cnt >= k) {
            // T*: each thread keeps its k best lower bounds (sorted, kk <= 16), then
            // k rounds pop the block's best thread head
            float tl[16];
            int ti[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                tl[q] = -INFINITY;
                ti[q] = INT_MAX;
            }
            for (int j = tid; j < cnt; j += BLOCK) {
                const float v = cand_lb[(int64_t)row * kCertCap + j];
                if (!ranks_above(v, j, tl[15], ti[15])) continue;
#pragma unroll
                for (int q = 15; q >= 0; --q) {  // insertion; tl[q - 1] is read before it moves
                    if (!ranks_above(v, j, tl[q], ti[q])) continue;
                    if (q > 0 && ranks_above(v, j, tl[q - 1], ti[q - 1])) {
                        tl[q] = tl[q - 1];
                        ti[q] = ti[q - 1];
                    } else {
                        tl[q] = v;
                        ti[q] = j;
                    }
                }
            }
            float kth = -INFINITY;
            for (int r = 0; r < k; ++r) {
                float ov;
                int oi;
                block_pick1(tl[0], ti[0], ov, oi);
                kth = ov;
                if (oi == ti[0] && oi != INT_MAX) {  // the winner pops its head (candidate ids are unique)
#pragma unroll
                    for (int q = 0; q < 15; ++q) {
                        tl[q] = tl[q + 1];
                        ti[q] = ti[q + 1];
                    }
                    tl[15] = -INFINITY;
                    ti[15] = INT_MAX;
                }
            }
            Tf = fmaxf(Tf, kth);
        }
        for (int j = tid; j < cnt; j += BLOCK)
            if (cand_ub[(int64_t)row * kCertCap + j] >= Tf) {
                const int p = atomicAdd(&s_n, 1);
                if (p < kSurv) s_i[p] = cand_idx[(int64_t)row * kCertCap + j];
            }
        __syncthreads();
        full = s_n > kSurv;  // uniform
        __syncthreads();     // every thread has read s_n before the fallback may rewrite it
        if (!full) {
            for (int j = w; j < s_n; j += BLOCK / 64) {
                const float v = wave_dot2(Uh + (int64_t)s_i[j] * d, xh, xl, d, lane);
                if (lane == 0) s_v[j] = v;
            }
            __syncthreads();
        }
    }
    if (full) {
        // overflow: one pass over the vocabulary, each wave keeping its k best
        // in lanes 0..k-1 (sorted), then the wave lists go to LDS
        float lv = -INFINITY;
        int li = INT_MAX;
        for (int v0 = w; v0 < V; v0 += BLOCK / 64) {
            const float v = wave_dot2(Uh + (int64_t)v0 * d, xh, xl, d, lane);
            const uint64_t above = __ballot(lane < k && ranks_above(v, v0, lv, li));
            if (above) {  // the lanes v ranks above form a suffix [pos, k)
                const int pos = __ffsll((long long)above) - 1;
                const float uv = __shfl_up(lv, 1, 64);
                const int ui = __shfl_up(li, 1, 64);
                if (lane > pos && lane < k) {
                    lv = uv;
                    li = ui;
                }
                if (lane == pos) {
                    lv = v;
                    li = v0;
                }
            }
        }
        if (lane < k) {
            s_v[w * 16 + lane] = lv;
            s_i[w * 16 + lane] = li;
        } else if (lane < 16) {
            s_v[w * 16 + lane] = -INFINITY;
            s_i[w * 16 + lane] = INT_MAX;
        }
        if (tid == 0) s_n = (BLOCK / 64) * 16;
        __syncthreads();
    }
    // k rounds of a block argmax over the re-scored values (at most kSurv)
    float out_v = -INFINITY;
    int out_i = INT_MAX;
    {
        float pv = INFINITY;
        int pi = -1;
        for (int r = 0; r < k; ++r) {
            float bv = -INFINITY;
            int bi = INT_MAX;
            for (int j = tid; j < s_n; j += BLOCK)
                if (ranks_above(pv, pi, s_v[j], s_i[j]) && ranks_above(s_v[j], s_i[j], bv, bi)) {
                    bv = s_v[j];
                    bi = s_i[j];
                }
            float ov;
            int oi;
            block_pick1(bv, bi, ov, oi);
            if (tid == r) {
                out_v = ov;
                out_i = oi;
            }
            pv = ov;
            pi = oi;
        }
    }
    if (tid < kmax) {
        const bool ok = tid < k && out_i != INT_MAX;
        const int64_t o = ((int64_t)m * nh + hh) * kmax + tid;
        topk_idx[o] = ok ? out_i : -1;
        topk_val[o] = ok ? out_v : -INFINITY;
    }
}

// The k-th largest of the wave's 64 values (one per lane) in the
// order-preserving int encoding: the largest t with at least k values >= t,
// built bit by bit from the top (32 ballots; cost independent of k).
__device__ __forceinline__ int wave_kth_largest_ordered(int v, int k) {
    const uint32_t u = (uint32_t)v ^ 0x80000000u;  // signed order -> unsigned order
    uint32_t res = 0u;
#pragma unroll
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t t = res | (1u << bit);
        if (__popcll(__ballot(u >= t)) >= k) res = t;
    }
    return (int)(res ^ 0x80000000u);
}

// The wide kernel's tiling with one product per term (hi) in three 24 KB
// stages, the tile's largest U row norm accumulated from the operand
// fragments, and the certified epilogue: per activation row, the bound E of
// this tile, a lower bound of the row's k-th best logit (atomicMax), and
// every entry that can still reach the top k appended to the row's candidate
// buffer. The epilogue's global atomics go out for all of a wave's columns at
// once rather than one column after another.
// PRE: the tiles' row norms come from a table made once per weight set
// (k_tile_norms) instead of the Gram products, 4 of every 36 MFMAs.
template <bool PRE>
__global__ __launch_bounds__(BLOCK, 2) void k_vocab_mfma_cert(const uint16_t* __restrict__ U,
                                                              const uint16_t* __restrict__ hhi, int M, int d, int V,
                                                              int nh, int head0, int vtiles, int mtiles, KW kk, int Mh,
                                                              const float* __restrict__ tile_n2,
                                                              const float* __restrict__ lo_norm,
                                                              const float* __restrict__ h_norm, float cert_c,
                                                              int* __restrict__ bound, int* __restrict__ slots,
                                                              int* __restrict__ count,
                                                              float* __restrict__ cand_ub, float* __restrict__ cand_lb,
                                                              int* __restrict__ cand_idx) {
    __shared__ __align__(1024) unsigned char sbuf0[CSTAGE];
    __shared__ __align__(1024) unsigned char sbuf1[CSTAGE];
    __shared__ __align__(1024) unsigned char sbuf2[CSTAGE];
    __shared__ float s_bound[VM];
    __shared__ float s_E[VM];
    __shared__ float s_nrm[4];
    const int units = nh * vtiles;
    int unit, mt;
    if (!decode_tile(blockIdx.x, mtiles, units, unit, mt)) return;
    // heads interleaved in dispatch order, so the first blocks to finish tighten every head's bounds
    const int hh = unit % nh, vt = unit / nh;
    const int v0 = vt * VR, m0 = mt * VM;
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int g4 = lane >> 4, c16 = lane & 15, wr = w >> 1, wc = w & 1;
    const int64_t hbase = (int64_t)hh * M * d;

    const int r0 = 16 * w + (lane >> 2);
    const uint32_t voff0 = (uint32_t)r0 * d * 2 + 16 * ((lane & 3) ^ ((r0 >> 1) & 3));
    const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(U + ((int64_t)(head0 + hh) * V + v0) * d), 0, min(V - v0, VR) * d * 2, RSRC3);
    const __amdgpu_buffer_rsrc_t rH =
        __builtin_amdgcn_make_buffer_rsrc((void*)(hhi + hbase + (int64_t)m0 * d), 0, min(M - m0, VM) * d * 2, RSRC3);
    auto issue = [&](int k0, unsigned char* base) {
#pragma unroll
        for (int j = 0; j < NPA; ++j) dmab(rA, base + (w + 4 * j) * 1024, voff0 + (uint32_t)(64 * j * d + k0) * 2);
#pragma unroll
        for (int j = 0; j < NPB; ++j) dmab(rH, base + A_BYTES + (w + 4 * j) * 1024, voff0 + (uint32_t)(64 * j * d + k0) * 2);
    };

    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Gram blocks A A^T of this wave's operand rows 16 (4 wc + j) .. + 15 (j < 4):
    // their diagonals are the squared row norms of U over the whole contraction
    f32x4 gram[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) gram[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int slot = (g4 ^ ((c16 >> 1) & 3)) * 16;
    auto compute = [&](const unsigned char* sA) {
        const unsigned char* sB = sA + A_BYTES;
        // the highest issue priority over the stage's fragment reads and
        // products: a wave whose stage has landed keeps the matrix units fed
        // while the SIMD's other wave waits (raised only after the reads,
        // the pass was slower)
        __builtin_amdgcn_s_setprio(3);
        bf16x8 a[8];
#pragma unroll
        for (int rb = 0; rb < 8; ++rb)
            a[rb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(sA + (128 * wr + 16 * rb + c16) * ROWB + slot));
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            const bf16x8 b =
                __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(sB + (64 * wc + 16 * cb + c16) * ROWB + slot));
#pragma unroll
            for (int rb = 0; rb < 8; ++rb)
                acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[rb], b, acc[rb][cb], 0, 0, 0);
        }
        // the two waves of a row band split its Gram blocks: wc takes row blocks 4 wc .. 4 wc + 3
        if constexpr (!PRE) {
            if (wc == 0) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    gram[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], a[j], gram[j], 0, 0, 0);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    gram[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[4 + j], a[4 + j], gram[j], 0, 0, 0);
            }
        }
        __builtin_amdgcn_s_setprio(0);
    };

    // Three stage buffers with two stages in flight, as in the narrow kernel:
    // the wait leaves the newer stage's loads (NPA + NPB per wave) open; the
    // barrier is LDS-only, so it does not wait for them either.
    const int nk = d / VK;
    constexpr int kStageLoads = NPA + NPB;  // buffer->LDS loads issue() makes per wave
    auto step = [&](int s, const unsigned char* cur, unsigned char* nxt) {
        __builtin_amdgcn_s_waitcnt(md_wave::waitcnt_vm(kStageLoads));
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        issue(min(s + 2, nk - 1) * VK, nxt);
        __builtin_amdgcn_sched_barrier(0);
        compute(cur);
    };
    issue(0, sbuf0);
    issue(min(1, nk - 1) * VK, sbuf1);
    int ks = 0;
    for (; ks + 3 <= nk; ks += 3) {
        step(ks, sbuf0, sbuf2);
        step(ks + 1, sbuf1, sbuf0);
        step(ks + 2, sbuf2, sbuf1);
    }
    if (ks < nk) step(ks, sbuf0, sbuf2);
    if (ks + 1 < nk) step(ks + 1, sbuf1, sbuf0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the repeated loads land before the buffers are reused
    // a half tile's logits: column c (row of h') takes 512 bytes in buffer c / 48
    auto colp = [&](int c) -> unsigned char* {
        unsigned char* bb = c < CCOLS ? sbuf0 : (c < 2 * CCOLS ? sbuf1 : sbuf2);
        return bb + (c % CCOLS) * 512;
    };
    // the tile's largest squared row norm (rows past V loaded nothing: norm 0).
    // Lane (g4, c16) holds Gram rows 4 g4 + i of column c16: the diagonal entry
    // when c16 - 4 g4 = i is in 0..3.
    {
        float mx = 0.f;
        const int di = c16 - 4 * g4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float dv = di == 0 ? gram[j][0] : di == 1 ? gram[j][1] : di == 2 ? gram[j][2] : di == 3 ? gram[j][3] : 0.f;
            mx = fmaxf(mx, dv);
        }
        mx = md_wave::wave_max(mx);
        if constexpr (PRE) mx = tile_n2[(int64_t)(head0 + hh) * vtiles + vt];
        if (lane == 0) s_nrm[w] = mx;
    }
    __syncthreads();
    if (tid < VM) {
        const int m = m0 + tid;
        if (m < M) {
            const float N = sqrtf(fmaxf(fmaxf(s_nrm[0], s_nrm[1]), fmaxf(s_nrm[2], s_nrm[3]))) * (1.f + 0x1p-10f);
            const int row = hh * M + m;
            s_E[tid] = N * ((1.f + 0x1p-7f) * lo_norm[row] + cert_c * h_norm[row]);
            s_bound[tid] = o2f(__hip_atomic_load(bound + row, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        } else {
            s_E[tid] = 0.f;
            s_bound[tid] = INFINITY;
        }
    }
    for (int h = 0; h < 2; ++h) {
        __syncthreads();
        if (wr == h) {
#pragma unroll
            for (int rb = 0; rb < 8; ++rb)
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) {
                    const int col = 64 * wc + 16 * cb + c16;
                    *reinterpret_cast<f32x4*>(colp(col) + (((4 * rb + g4) ^ (col & 15)) * 16)) = acc[rb][cb];
                }
        }
        __syncthreads();
        const int vh = v0 + 128 * h;
        // Lane i owns column w + 4 i (i < 32). Pass 1 reads the tile from LDS
        // only: per column, the entries that may reach the top k (>= lim) and
        // their best. The global atomics of all columns then go out together.
        auto load2 = [&](int col, float (&x)[2]) {
            const unsigned char* Sc = colp(col);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int rr = lane + 64 * e;
                x[e] = vh + rr < V ? *reinterpret_cast<const float*>(Sc + (((rr >> 2) ^ (col & 15)) * 16) + (rr & 3) * 4)
                                   : -INFINITY;
            }
        };
        float my_best = -INFINITY, my_lim = INFINITY, my_E = 0.f;
        int my_cnt = 0;
        for (int i = 0; i < 32; ++i) {
            const int col = w + 4 * i;
            if (m0 + col >= M) break;  // uniform: columns past M are padding
            const float E = s_E[col];
            const float lim = s_bound[col] - E;  // entries below cannot reach the top k
            float x0[2];
            load2(col, x0);
            int cnt = 0;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                if (x0[e] < lim) x0[e] = -INFINITY;
                cnt += __popcll(__ballot(x0[e] != -INFINITY));
            }
            float best = fmaxf(x0[0], x0[1]);
            best = md_wave::wave_max(best);
            if (lane == i) {
                my_best = best;
                my_cnt = cnt;
                my_lim = lim;
                my_E = E;
            }
        }
        // This half tile's best entry is within E of a logit it bounds from
        // below: it raises slot (half-tile id % 64) of the row. The k-th largest
        // slot comes from k distinct entries, so it bounds the row's k-th best
        // logit from below; it only moves when a slot does.
        const int my_row = hh * M + m0 + w + 4 * lane;
        bool rose = false;
        if (lane < 32 && my_cnt > 0) {
            const int nv = f2o(my_best - my_E);
            const int old = atomicMax(slots + (int64_t)my_row * kSlots + ((2 * vt + h) & (kSlots - 1)), nv);
            rose = nv > old;
            // a slot value at or below the bound read at the tile's start cannot raise the bound
            rose = rose && (my_best - my_E > my_lim + my_E);
        }
        float my_thr = my_lim;
        // The k-th largest slot of every column whose slot rose: the slot rows
        // of up to 8 columns are loaded together (one memory round trip), then
        // each is reduced by a bit search (k > 2) or k rounds of a wave argmax.
        for (uint64_t rm = __ballot(rose); rm;) {
            int ids[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                ids[q] = rm ? __ffsll((long long)rm) - 1 : -1;
                rm &= rm ? rm - 1 : 0ull;
            }
            float svs[8];
#pragma unroll
            for (int q = 0; q < 8; ++q)
                svs[q] = ids[q] >= 0 ? o2f(__hip_atomic_load(slots + (int64_t)(hh * M + m0 + w + 4 * ids[q]) * kSlots + lane,
                                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
                                     : -INFINITY;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                if (ids[q] < 0) break;  // uniform
                const int i = ids[q];
                const int m = m0 + w + 4 * i, row = hh * M + m;
                const int k = (Mh > 0 ? kk.at(__builtin_amdgcn_readfirstlane(min(m / Mh, 7))) : kk.at(hh));
                float sv = svs[q];
                float kth = -INFINITY;
                if (k > 2) kth = o2f(wave_kth_largest_ordered(f2o(sv), k));
                for (int r = 0; k <= 2 && r < k; ++r) {
                    float bv = sv;
                    int bl = lane;
                    md_wave::wave_argmax(bv, bl);
                    kth = bv;
                    if (bl == lane) sv = -INFINITY;
                }
                if (kth != -INFINITY) {
                    if (lane == 0) atomicMax(bound + row, f2o(kth));
                    if (lane == i) my_thr = fmaxf(my_thr, kth - my_E);
                }
            }
        }
        // per column, the entries >= thr (value + E is their upper bound): count, reserve, write
        uint64_t my_b0 = 0ull, my_b1 = 0ull;
        const uint64_t with = __ballot(lane < 32 && my_cnt > 0);
        for (uint64_t cm = with; cm; cm &= cm - 1) {
            const int i = __ffsll((long long)cm) - 1;
            const int col = w + 4 * i;
            const float thr = __shfl(my_thr, i, 64), lim = __shfl(my_lim, i, 64);
            float x0[2];
            load2(col, x0);
            // rows past V read as -inf and never qualify, whatever lim and thr are
            const uint64_t b0 = __ballot(x0[0] != -INFINITY && x0[0] >= lim && x0[0] >= thr);
            const uint64_t b1 = __ballot(x0[1] != -INFINITY && x0[1] >= lim && x0[1] >= thr);
            if (lane == i) {
                my_b0 = b0;
                my_b1 = b1;
            }
        }
        int my_base = 0;
        const int my_n = __popcll(my_b0) + __popcll(my_b1);
        if (my_n > 0) my_base = atomicAdd(count + my_row, my_n);
        const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        for (uint64_t cm = __ballot(my_n > 0); cm; cm &= cm - 1) {
            const int i = __ffsll((long long)cm) - 1;
            const int col = w + 4 * i, row = hh * M + m0 + col;
            const uint64_t b0 = __shfl(my_b0, i, 64), b1 = __shfl(my_b1, i, 64);
            const int base = __shfl(my_base, i, 64);
            const float E = __shfl(my_E, i, 64);
            float x0[2];
            load2(col, x0);
            const int n0 = __popcll(b0);
            if ((b0 >> lane) & 1) {
                const int p = base + __popcll(b0 & below);
                if (p < kCertCap) {
                    cand_ub[(int64_t)row * kCertCap + p] = x0[0] + E;
                    cand_lb[(int64_t)row * kCertCap + p] = x0[0] - E;
                    cand_idx[(int64_t)row * kCertCap + p] = vh + lane;
                }
            }
            if ((b1 >> lane) & 1) {
                const int p = base + n0 + __popcll(b1 & below);
                if (p < kCertCap) {
                    cand_ub[(int64_t)row * kCertCap + p] = x0[1] + E;
                    cand_lb[(int64_t)row * kCertCap + p] = x0[1] - E;
                    cand_idx[(int64_t)row * kCertCap + p] = vh + lane + 64;
                }
            }
        }
    }
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The residual over many rows (Medusa heads on every node of a batch): the
// same GEMM shape as the certified pass, so the same pipeline. Block tile 256
// rows of W x 128 activation rows, 4 waves of 128 x 64 (8 x 4 MFMA tiles),
// stages of 24 KB (W 16 KB, h 8 KB) by buffer->LDS loads into three named
// buffers with two in flight, the 64-byte LDS rows swizzled as there; one
// product (h is exact in bf16). The epilogue applies h' = h + SiLU(z + b)
// per 4 outputs of a lane. Tiles never straddle heads (d % 256 == 0).
__global__ __launch_bounds__(BLOCK, 2) void k_residual_wide(const uint16_t* __restrict__ W,
                                                            const uint16_t* __restrict__ bias, GemmRows rows, int M,
                                                            int d, int nh, int head0, int mtiles,
                                                            float* __restrict__ hres, float* __restrict__ hres_out,
                                                            uint16_t* __restrict__ hhi, uint16_t* __restrict__ hlo,
                                                            int* __restrict__ bound) {
    __shared__ __align__(1024) unsigned char wbuf0[CSTAGE];
    __shared__ __align__(1024) unsigned char wbuf1[CSTAGE];
    __shared__ __align__(1024) unsigned char wbuf2[CSTAGE];
    const int units = nh * (d / VR);
    int unit, mt;
    if (!decode_tile(blockIdx.x, mtiles, units, unit, mt)) return;
    const int row0 = unit * VR;  // over nh * d rows
    const int hh = row0 / d, rt0 = row0 - hh * d;
    const int m0 = mt * VM;
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = lane >> 4, c16 = lane & 15, wr = w >> 1, wc = w & 1;

    // the vocabulary kernel that follows keeps a lower bound of each (head, row)'s
    // k-th best logit here; start from -inf
    if (blockIdx.x == 0)
        for (int j = tid; j < nh * M; j += BLOCK) bound[j] = f2o(-INFINITY);

    const int r0 = 16 * w + (lane >> 2);
    const uint32_t voff0 = (uint32_t)r0 * d * 2 + 16 * ((lane & 3) ^ ((r0 >> 1) & 3));
    const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(W + ((int64_t)head0 * d + row0) * d), 0, VR * d * 2, RSRC3);
    const __amdgpu_buffer_rsrc_t rH = __builtin_amdgcn_make_buffer_rsrc((void*)(rows.h + (int64_t)m0 * d), 0,
                                                                        min(M - m0, VM) * d * 2, RSRC3);
    auto issue = [&](int k0, unsigned char* base) {
#pragma unroll
        for (int j = 0; j < NPA; ++j) dmab(rA, base + (w + 4 * j) * 1024, voff0 + (uint32_t)(64 * j * d + k0) * 2);
#pragma unroll
        for (int j = 0; j < NPB; ++j) dmab(rH, base + A_BYTES + (w + 4 * j) * 1024, voff0 + (uint32_t)(64 * j * d + k0) * 2);
    };
    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int slot = (g4 ^ ((c16 >> 1) & 3)) * 16;
    auto compute = [&](const unsigned char* sA) {
        const unsigned char* sB = sA + A_BYTES;
        bf16x8 a[8];
#pragma unroll
        for (int rb = 0; rb < 8; ++rb)
            a[rb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(sA + (128 * wr + 16 * rb + c16) * ROWB + slot));
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            const bf16x8 b =
                __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(sB + (64 * wc + 16 * cb + c16) * ROWB + slot));
#pragma unroll
            for (int rb = 0; rb < 8; ++rb)
                acc[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[rb], b, acc[rb][cb], 0, 0, 0);
        }
    };
    // the certified pass's schedule: the wait leaves the newer stage's NPA + NPB
    // loads per wave open; an LDS-only barrier; past the last stage the loads
    // repeat it
    const int nk = d / VK;
    constexpr int kStageLoads = NPA + NPB;  // buffer->LDS loads issue() makes per wave
    auto step = [&](int s, const unsigned char* cur, unsigned char* nxt) {
        __builtin_amdgcn_s_waitcnt(md_wave::waitcnt_vm(kStageLoads));
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        issue(min(s + 2, nk - 1) * VK, nxt);
        __builtin_amdgcn_sched_barrier(0);
        compute(cur);
    };
    issue(0, wbuf0);
    issue(min(1, nk - 1) * VK, wbuf1);
    int ks = 0;
    for (; ks + 3 <= nk; ks += 3) {
        step(ks, wbuf0, wbuf2);
        step(ks + 1, wbuf1, wbuf0);
        step(ks + 2, wbuf2, wbuf1);
    }
    if (ks < nk) step(ks, wbuf0, wbuf2);
    if (ks + 1 < nk) step(ks + 1, wbuf1, wbuf0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the repeated loads land before the block ends

    // lane holds z[row rt0 + 128 wr + 16 rb + 4 g4 + i][activation row m0 + 64 wc + 16 cb + c16].
    // The epilogue's loads go out in batches (the 8 bias pairs once, then a
    // column block's 8 base pairs) before the values that use them: 4 memory
    // round trips per lane instead of one per 4 outputs.
    u32x2 bw[8];
#pragma unroll
    for (int rb = 0; rb < 8; ++rb) bw[rb] = bias_words(bias, head0, hh, d, rt0 + 128 * wr + 16 * rb + 4 * g4);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        const int m = m0 + 64 * wc + 16 * cb + c16;
        if (m >= M) continue;
        u32x2 hw[8];
#pragma unroll
        for (int rb = 0; rb < 8; ++rb)
            hw[rb] = *reinterpret_cast<const u32x2*>(rows.h + (int64_t)m * d + rt0 + 128 * wr + 16 * rb + 4 * g4);
#pragma unroll
        for (int rb = 0; rb < 8; ++rb)
            residual_out_w(acc[rb][cb], bw[rb], hw[rb], M, d, hh, m, rt0 + 128 * wr + 16 * rb + 4 * g4, hres,
                           hres_out, hhi, hlo, BoOut{nullptr, nullptr, 0, 0});
    }
}

__global__ void k_fill_bound(int* __restrict__ bound, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) bound[i] = f2o(-INFINITY);
}

}  // namespace

// With an operand-order copy of the LM head, 2 to 7 rows run on the matrix
// cores too (the few-row kernels then read at the streaming rate).
bool argmax_mfma_applicable(int dt, int R, int d, bool op) {
    return dt == 1 && (R >= 8 || (op && R >= 2 && R <= kNarrowRows)) && d % (2 * VK) == 0;
}

size_t argmax_mfma_ws_bytes(int R, int V) {
    const size_t vtiles = (size_t)(V + VR - 1) / VR;
    return 2 * align256((size_t)R * 2 * vtiles * 4) + align256((size_t)R * 4);
}

// The target's choice per row: one bf16 product per term (hidden states and
// LM head are exact in bf16), the same epilogue with k = 1; the caller merges
// the lists (two per vocabulary tile).
hipError_t argmax_mfma_launch(int R, int d, int V, const void* H, const void* Wt, const void* Wt_op, void* ws,
                              hipStream_t s, float** part_val, int** part_idx, int* nlists) {
    const int vtiles = (V + VR - 1) / VR, vmtiles = (R + VM - 1) / VM;
    char* w = reinterpret_cast<char*>(ws);
    float* pv = reinterpret_cast<float*>(w);
    w += align256((size_t)R * 2 * vtiles * 4);
    int* pi = reinterpret_cast<int*>(w);
    w += align256((size_t)R * 2 * vtiles * 4);
    int* bound = reinterpret_cast<int*>(w);
    hipLaunchKernelGGL(k_fill_bound, dim3((R + 255) / 256), dim3(256), 0, s, bound, R);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    KW kk;
    for (int i = 0; i < 8; ++i) kk.v[i] = 1;
    const uint16_t* h = reinterpret_cast<const uint16_t*>(H);
    const bool op = Wt_op != nullptr;
    const uint16_t* wt = reinterpret_cast<const uint16_t*>(op ? Wt_op : Wt);
    if (R <= kNarrowRows) {
        if (R > NM) {
            const int cb = (R + 15) / 16;
            err = op ? launch_direct<1, true, false>(cb, dim3(vtiles), s, wt, h, h, R, d, V, 1, 0, vtiles, 1, kk, 0, pv,
                                                     pi, bound)
                     : launch_direct<1, false, false>(cb, dim3(vtiles), s, wt, h, h, R, d, V, 1, 0, vtiles, 1, kk, 0, pv,
                                                      pi, bound);
            if (err != hipSuccess) return err;
        } else {
            const dim3 grid(8 * ((vtiles + 7) / 8));
            if (op)
                hipLaunchKernelGGL((k_vocab_mfma_narrow<1, true, false>), grid, dim3(BLOCK), 0, s, wt, h, h, R, d, V, 1, 0,
                                   vtiles, 1, 1, kk, 0, pv, pi, bound, nullptr, nullptr);
            else
                hipLaunchKernelGGL((k_vocab_mfma_narrow<1, false, false>), grid, dim3(BLOCK), 0, s, wt, h, h, R, d, V, 1,
                                   0, vtiles, 1, 1, kk, 0, pv, pi, bound, nullptr, nullptr);
        }
        *nlists = vtiles;
    } else {  // row-major LM head: the many-row kernel stages its tiles through LDS
        hipLaunchKernelGGL(k_vocab_mfma<1>, dim3(8 * vmtiles * ((vtiles + 7) / 8)), dim3(BLOCK), 0, s,
                           reinterpret_cast<const uint16_t*>(Wt), h, h, R, d, V,
                           1, 0, vtiles, vmtiles, 1, kk, 0, pv, pi, bound);
        *nlists = 2 * vtiles;
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
    *part_val = pv;
    *part_idx = pi;
    return hipSuccess;
}

namespace {
// One thread per 16-byte chunk of the operand-order copy.
__global__ __launch_bounds__(BLOCK) void k_operand_order(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                                         int rows, int cols, int tiles, int64_t chunks) {
    const int ks = cols / VK;
    for (int64_t i = (int64_t)blockIdx.x * BLOCK + threadIdx.x; i < chunks; i += (int64_t)gridDim.x * BLOCK) {
        int64_t q = i;
        const int lane = (int)(q % 64);
        q /= 64;
        const int rb = (int)(q % (OP_TILE / 16));
        q /= OP_TILE / 16;
        const int step = (int)(q % ks);
        q /= ks;
        const int t = (int)(q % tiles);
        const int64_t mat = q / tiles;
        const int row = t * OP_TILE + rb * 16 + (lane & 15);
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (row < rows)
            v = *reinterpret_cast<const u32x4*>(src + (mat * rows + row) * cols + step * VK + 8 * (lane >> 4));
        *reinterpret_cast<u32x4*>(dst + i * 8) = v;
    }
}
}  // namespace

// c(d) of the certified pass's bound E (see the comment above kCertCap),
// rounded up to float.
float cert_rounding_allowance(int d) {
    if (d <= 0) return 0.f;
    const double u = 0x1p-24;
    auto gamma = [u](double n) { return n * u / (1.0 - n * u); };
    const double n_mfma = d / 32.0 + 32.0, n_rescore = d / 64.0 + 6.0;
    const double c = (gamma(n_mfma) * (1.0 + 0x1p-8) + gamma(n_rescore) * (1.0 + 0x1p-16)) * (1.0 + 0x1p-10);
    const float f = (float)c;
    return (double)f >= c ? f : nextafterf(f, INFINITY);
}

size_t operand_order_bytes(int nmat, int rows, int cols) {
    return (size_t)nmat * ((rows + OP_TILE - 1) / OP_TILE) * OP_TILE * cols * 2;
}

hipError_t operand_order_launch(int nmat, int rows, int cols, const void* src, void* dst, hipStream_t s) {
    const int tiles = (rows + OP_TILE - 1) / OP_TILE;
    const int64_t chunks = (int64_t)nmat * tiles * OP_TILE * cols / 8;
    const int64_t blocks = std::min<int64_t>((chunks + BLOCK - 1) / BLOCK, 8 * device_cus());
    hipLaunchKernelGGL(k_operand_order, dim3((unsigned)blocks), dim3(BLOCK), 0, s, reinterpret_cast<const uint16_t*>(src),
                       reinterpret_cast<uint16_t*>(dst), rows, cols, tiles, chunks);
    return hipGetLastError();
}

bool heads_mfma_applicable(int dt, int M, int d, int din, bool op, int rows_v) {
    // d % 128: whole residual tiles, and an even number of vocabulary stages;
    // with an operand-order copy of U from 2 projection columns (rows_v: the
    // rows, or heads x rows through one shared projection; the GEMV stays
    // for 1)
    return dt == 1 && (M >= 8 || (op && rows_v >= 2)) && d % TR == 0 && din % KS == 0 && d % (2 * VK) == 0;
}

// Contraction chunks of the residual: enough (tile, chunk) blocks for two per
// CU of a 256-CU part, each chunk a whole number of K steps (a power of two
// dividing din / KS).
int residual_ksplit(int M, int d, int din, int nh) {
    const int blocks = ((M + TM - 1) / TM) * (nh * d / TR);
    int ks = 1;
    while (blocks * ks < 512 && (din / KS) % (2 * ks) == 0 && 2 * ks <= 64) ks *= 2;
    return ks;
}

// Up to 16 activation rows: k_residual_rows (16 rows of W a block, the whole
// contraction, no split partials), where every gathered row offset fits the
// 31-bit range its buffer loads address (E: V x d bf16).
bool residual_rows(int M, int d, int din, int V) {
    return M >= 1 && M <= 16 && din % 2048 == 0 && d % 16 == 0 && (din == d || (int64_t)V * d * 2 <= 0x7FF00000LL);
}

// 17 to 77 activation rows at din = 8,192: k_residual_staged (the activation
// chunk staged in LDS, 8 contraction chunks, k_residual_finish after it).
bool residual_staged(int M, int d, int din, int nh) {
    return M > 16 && M < kStageRows && din == 8 * kStageKC && d % 128 == 0 && (nh * d / 128) * 8 >= 256;
}

// Many Medusa rows with whole 256-row tiles of W and enough of them to fill
// the GPU without a split contraction: the certified pass's pipeline
// (k_residual_wide); otherwise the 128 x 128 register-staged tiles.
bool residual_wide(int kind, int M, int d, int din, int nh) {
    return kind == 0 && din == d && M > kNarrowRows && d % VR == 0 && residual_ksplit(M, d, din, nh) == 1;
}

// Workspace: h' (float32, hi, lo), the per-row bounds, the split-contraction
// partials, then either the narrow kernel's partial lists and hi / lo in its
// operand order or the certified pass's norms, slots and candidate buffers.
struct MfmaWs {
    float* hres;
    uint16_t *hhi, *hlo;
    int* bound;
    float* zpart;
    float *pv;  // narrow: partial lists [rows][vtiles][kmax]
    int* pi;
    uint16_t *bo_hi, *bo_lo;  // narrow: hi / lo in its activation operand order (BoOut)
    float *lo_norm, *h_norm;  // certified: per row
    int *count, *slots;
    float *cand_ub, *cand_lb;
    int* cand_idx;
    size_t bytes;
};

MfmaWs mfma_ws_layout(char* base, int M, int d, int din, int V, int nh, int kmax, bool certified) {
    MfmaWs L = {};
    size_t off = 0;
    auto take = [&](size_t n) {
        char* p = base ? base + off : nullptr;
        off += align256(n);
        return p;
    };
    const size_t e = (size_t)nh * M * d, rows = (size_t)nh * M;
    const int ks = residual_rows(M, d, din, V) ? 1 : (residual_staged(M, d, din, nh) ? 8 : residual_ksplit(M, d, din, nh));
    L.hres = reinterpret_cast<float*>(take(e * 4));
    L.hhi = reinterpret_cast<uint16_t*>(take(e * 2));
    L.hlo = reinterpret_cast<uint16_t*>(take(e * 2));
    L.bound = reinterpret_cast<int*>(take(rows * 4));
    L.zpart = ks > 1 ? reinterpret_cast<float*>(take((size_t)ks * e * 4)) : nullptr;
    if (!certified) {
        const size_t lists = rows * (size_t)((V + VR - 1) / VR) * kmax * 4;
        L.pv = reinterpret_cast<float*>(take(lists));
        L.pi = reinterpret_cast<int*>(take(lists));
        // per head whole 64-row tiles (also covers the heads' rows as one matrix)
        const size_t bo = (size_t)nh * ((M + kBoTile - 1) / kBoTile) * kBoTile * d * 2;
        L.bo_hi = reinterpret_cast<uint16_t*>(take(bo));
        L.bo_lo = reinterpret_cast<uint16_t*>(take(bo));
    } else {
        L.lo_norm = reinterpret_cast<float*>(take(rows * 4));
        L.h_norm = reinterpret_cast<float*>(take(rows * 4));
        L.count = reinterpret_cast<int*>(take(rows * 4));
        L.slots = reinterpret_cast<int*>(take(rows * kSlots * 4));
        L.cand_ub = reinterpret_cast<float*>(take(rows * kCertCap * 4));
        L.cand_lb = reinterpret_cast<float*>(take(rows * kCertCap * 4));
        L.cand_idx = reinterpret_cast<int*>(take(rows * kCertCap * 4));
    }
    L.bytes = off;
    return L;
}

// The certified pass runs when the vocabulary GEMM sees more than
// kNarrowRows rows, and only if its bounds can work: the vocabulary tiles of
// one (head, row tile) that run in the first round of resident blocks (two a
// CU) all start from an empty bound, and their entries (2 x 128 half-tile
// columns each) must fit the candidate buffer; past that the exact fallback
// scan would take over. Other shapes run the two-product narrow kernel.
bool use_certified(int M, int V, int nh, int shared_u) {
    const int rows = shared_u ? nh * M : M, nh_u = shared_u ? 1 : nh;
    if (rows <= kNarrowRows) return false;
    const int vtiles = (V + VR - 1) / VR, mtiles = (rows + VM - 1) / VM;
    const int first_round = (2 * device_cus() + nh_u * mtiles - 1) / (nh_u * mtiles);
    return std::min(vtiles, first_round) * 2 * VM <= kCertCap;
}

size_t heads_mfma_ws_bytes(int M, int d, int din, int V, int nh, int kmax, int shared_u) {
    return mfma_ws_layout(nullptr, M, d, din, V, nh, kmax, use_certified(M, V, nh, shared_u)).bytes;
}

// Launches phase 1 and phase 2. With few rows the caller merges the lists
// (*nlists of them per row); with many rows the certified pass writes the
// top-k lists itself (*nlists = 0).
hipError_t heads_mfma_launch(const HeadsArgs& a, const DevTree* tree, hipStream_t s, hipEvent_t ev0, hipEvent_t ev1,
                             float** part_val, int** part_idx, int* nlists) {
    const int vtiles = (a.V + VR - 1) / VR;
    const int mtiles = (a.M + TM - 1) / TM;
    const bool cert = use_certified(a.M, a.V, a.nh, a.shared_u);
    const MfmaWs L = mfma_ws_layout(reinterpret_cast<char*>(a.ws), a.M, a.d, a.din, a.V, a.nh, a.kmax, cert);
    const size_t e = (size_t)a.nh * a.M * a.d, crow = (size_t)a.nh * a.M;
    KW kk;
    for (int i = 0; i < 8; ++i) kk.v[i] = i < a.nh ? a.kk[i] : 1;
    hipError_t err;
    if (cert) {
        hipLaunchKernelGGL(k_cert_prep, dim3((unsigned)((crow * kSlots + 255) / 256)), dim3(256), 0, s, L.bound, L.slots,
                           L.count, (int)crow);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }

    GemmRows rows;
    rows.kind = a.kind;
    rows.P = 1;
    rows.N = tree ? tree->n : 0;
    rows.V = a.V;
    for (int i = 0; i < 64; ++i) rows.parents[i] = 0;
    if (a.kind == 1) {
        const int off = tree->level_off[a.level];
        rows.P = tree->level_off[a.level + 1] - off;
        for (int j = 0; j < rows.P; ++j) rows.parents[j] = tree->lp[off + j];
    }
    rows.h = reinterpret_cast<const uint16_t*>(a.h);
    rows.E = reinterpret_cast<const uint16_t*>(a.E);
    rows.root_tok = a.root_tok;
    rows.tree_tok = a.tree_tok;

    const int units1 = a.nh * a.d / TR;
    const bool rows16 = residual_rows(a.M, a.d, a.din, a.V);
    const bool staged = !rows16 && residual_staged(a.M, a.d, a.din, a.nh);
    const int ksplit = rows16 ? 1 : (staged ? 8 : residual_ksplit(a.M, a.d, a.din, a.nh));
    const uint16_t* bias = reinterpret_cast<const uint16_t*>(a.b);
    // one Medusa row (a shared projection) with an operand-order copy: the GEMV residual
    // (one pass over W, HBM-bound) writes h' and its hi/lo split for the
    // matrix-core vocabulary kernel; otherwise a matrix-core residual
    const bool on_gemv = residual_on_gemv(a.dt, a.kind, a.M, a.d, a.din, a.U_op != nullptr);
    // the few-row vocabulary kernels read hi / lo in their operand order when
    // the matrix-core residual (k_residual_mfma, k_residual_finish) writes them
    const int rows_v = a.shared_u ? a.nh * a.M : a.M, nh_u = a.shared_u ? 1 : a.nh;
    const bool use_bo = !cert && !on_gemv && !residual_wide(a.kind, a.M, a.d, a.din, a.nh);
    const BoOut bo = use_bo ? BoOut{L.bo_hi, L.bo_lo, a.shared_u, a.nh} : BoOut{nullptr, nullptr, 0, 0};
    if (on_gemv) {
        float ninf = -INFINITY;
        int nb;
        memcpy(&nb, &ninf, 4);
        nb = nb >= 0 ? nb : nb ^ 0x7FFFFFFF;  // the bounds' order-preserving encoding of -inf
        if ((err = residual_gemv_split(a, tree, L.hres, L.hhi, L.hlo, L.bound, nb, s)) != hipSuccess) return err;
    } else if (residual_wide(a.kind, a.M, a.d, a.din, a.nh)) {
        const int wm = (a.M + VM - 1) / VM, wu = a.nh * (a.d / VR);
        hipLaunchKernelGGL(k_residual_wide, dim3(8 * wm * ((wu + 7) / 8)), dim3(BLOCK), 0, s,
                           reinterpret_cast<const uint16_t*>(a.W), bias, rows, a.M, a.d, a.nh, a.head0, wm, L.hres,
                           a.h_res, L.hhi, L.hlo, L.bound);
    } else if (rows16) {
        const dim3 g((unsigned)(a.nh * a.d / 16)), blk(kRowsWaves * MD_WAVE);
        if (a.W_op)
            hipLaunchKernelGGL((k_residual_rows<1, true>), g, blk, 0, s, reinterpret_cast<const uint16_t*>(a.W_op), bias,
                               rows, a.M, a.d, a.din, a.nh, a.head0, L.hres, a.h_res, L.hhi, L.hlo, L.bound, bo);
        else
            hipLaunchKernelGGL((k_residual_rows<1, false>), g, blk, 0, s, reinterpret_cast<const uint16_t*>(a.W), bias,
                               rows, a.M, a.d, a.din, a.nh, a.head0, L.hres, a.h_res, L.hhi, L.hlo, L.bound, bo);
    } else if (staged) {
        const dim3 g((unsigned)(8 * (a.nh * a.d / 128))), blk(kRowsWaves * MD_WAVE);
        const bool wop = a.W_op != nullptr;
        const uint16_t* Wp = reinterpret_cast<const uint16_t*>(wop ? a.W_op : a.W);
#define MD_STAGED(RCV)                                                                                                 \
    if (wop)                                                                                                           \
        hipLaunchKernelGGL((k_residual_staged<RCV, true>), g, blk, 0, s, Wp, rows, a.M, a.d, a.din, a.nh, a.head0,      \
                           L.zpart, L.bound);                                                                          \
    else                                                                                                               \
        hipLaunchKernelGGL((k_residual_staged<RCV, false>), g, blk, 0, s, Wp, rows, a.M, a.d, a.din, a.nh, a.head0,     \
                           L.zpart, L.bound)
        switch ((a.M + 15) / 16) {
            case 2: MD_STAGED(2); break;
            case 3: MD_STAGED(3); break;
            case 4: MD_STAGED(4); break;
            default: MD_STAGED(5); break;
        }
#undef MD_STAGED
    } else {
        hipLaunchKernelGGL(k_residual_mfma, dim3(ksplit * 8 * mtiles * ((units1 + 7) / 8)), dim3(BLOCK), 0, s,
                           reinterpret_cast<const uint16_t*>(a.W), bias, rows, a.M, a.d, a.din, a.nh, a.head0, mtiles,
                           ksplit, L.zpart, L.hres, a.h_res, L.hhi, L.hlo, L.bound, bo);
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (!on_gemv && ksplit > 1 && !residual_wide(a.kind, a.M, a.d, a.din, a.nh)) {
        const int64_t quads = e / 4;
        hipLaunchKernelGGL(k_residual_finish, dim3((unsigned)((quads + BLOCK - 1) / BLOCK)), dim3(BLOCK), 0, s, L.zpart,
                           ksplit, bias, rows, a.M, a.d, a.nh, a.head0, L.hres, a.h_res, L.hhi, L.hlo, bo);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (cert) {
        hipLaunchKernelGGL(k_row_norms, dim3((unsigned)((crow + 3) / 4)), dim3(BLOCK), 0, s, L.hres, (int)crow, a.d,
                           L.lo_norm, L.h_norm);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (ev0 && (err = hipEventRecord(ev0, s)) != hipSuccess) return err;
    // a shared projection is one matrix over the heads' nh * M rows
    const int units2 = nh_u * vtiles;
    const uint16_t* U = reinterpret_cast<const uint16_t*>(a.U);
    const int head0 = a.shared_u ? 0 : a.head0, Mh = a.shared_u ? a.M : 0;
    if (!cert) {  // few rows: HBM-bound, two products and the deeper pipeline
        // 65 to 128 rows: one register-streamed tile; otherwise 64-row tiles
        // (more than 128 rows only where the certified pass cannot work). With
        // an operand-order copy of U both read that instead.
        const bool op = a.U_op != nullptr;
        const uint16_t* UA = op ? reinterpret_cast<const uint16_t*>(a.U_op) : U;
        if (rows_v > NM && rows_v <= kNarrowRows) {
            const int cb = (rows_v + 15) / 16;
#define MD_DIRECT_L(OPV, BOV)                                                                                    \
    launch_direct<2, OPV, BOV>(cb, dim3(units2), s, UA, L.hhi, L.hlo, rows_v, a.d, a.V, nh_u, head0, vtiles, a.kmax, kk, \
                               Mh, L.pv, L.pi, L.bound, bo.hi, bo.lo)
            err = op ? (use_bo ? MD_DIRECT_L(true, true) : MD_DIRECT_L(true, false))
                     : (use_bo ? MD_DIRECT_L(false, true) : MD_DIRECT_L(false, false));
#undef MD_DIRECT_L
            if (err != hipSuccess) return err;
        } else {
            const int nmt = (rows_v + NM - 1) / NM;
            const dim3 grid(8 * nmt * ((units2 + 7) / 8));
#define MD_NARROW(OPV, BOV)                                                                                          \
    hipLaunchKernelGGL((k_vocab_mfma_narrow<2, OPV, BOV>), grid, dim3(BLOCK), 0, s, UA, L.hhi, L.hlo, rows_v, a.d, a.V, \
                       nh_u, head0, vtiles, nmt, a.kmax, kk, Mh, L.pv, L.pi, L.bound, bo.hi, bo.lo)
            if (op && use_bo)
                MD_NARROW(true, true);
            else if (op)
                MD_NARROW(true, false);
            else if (use_bo)
                MD_NARROW(false, true);
            else
                MD_NARROW(false, false);
#undef MD_NARROW
        }
        *nlists = vtiles;
    } else {  // many rows: one product and the certificate
        const int vmtiles = (rows_v + VM - 1) / VM;
        const dim3 cgrid(8 * vmtiles * ((units2 + 7) / 8));
        if (a.U_norms)
            hipLaunchKernelGGL(k_vocab_mfma_cert<true>, cgrid, dim3(BLOCK), 0, s, U, L.hhi, rows_v, a.d, a.V, nh_u, head0,
                               vtiles, vmtiles, kk, Mh, a.U_norms, L.lo_norm, L.h_norm, cert_rounding_allowance(a.d),
                               L.bound, L.slots, L.count, L.cand_ub, L.cand_lb, L.cand_idx);
        else
            hipLaunchKernelGGL(k_vocab_mfma_cert<false>, cgrid, dim3(BLOCK), 0, s, U, L.hhi, rows_v, a.d, a.V, nh_u,
                               head0, vtiles, vmtiles, kk, Mh, nullptr, L.lo_norm, L.h_norm,
                               cert_rounding_allowance(a.d), L.bound, L.slots, L.count, L.cand_ub, L.cand_lb,
                               L.cand_idx);
        *nlists = 0;
    }
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (ev1 && (err = hipEventRecord(ev1, s)) != hipSuccess) return err;
    if (cert) {
        hipLaunchKernelGGL(k_rescore, dim3((unsigned)crow), dim3(BLOCK), 0, s, U, L.hhi, L.hlo, a.M, a.d, a.V, a.nh,
                           a.head0, a.shared_u, kk, a.kmax, L.bound, L.count, L.cand_ub, L.cand_lb, L.cand_idx,
                           a.topk_idx, a.topk_val);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    *part_val = L.pv;
    *part_idx = L.pi;
    return hipSuccess;
}

int vocab_tiles(int V) { return (V + VR - 1) / VR; }

hipError_t vocab_tile_norms_launch(const void* U, int nmat, int V, int d, float* out, hipStream_t s) {
    const int vt = vocab_tiles(V);
    hipLaunchKernelGGL(k_tile_norms, dim3((unsigned)(nmat * vt)), dim3(BLOCK), 0, s,
                       reinterpret_cast<const uint16_t*>(U), V, d, vt, out);
    return hipGetLastError();
}
