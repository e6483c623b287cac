/*
 * Seeded synthetic inputs shared by the CPU oracle and the GPU path.
 *
 * This file holds no arithmetic of the decode step itself: it only turns
 * (seed, stream, element index) into numbers. Every tensor of a workload is
 * filled from its own stream, so any element can be regenerated on its own.
 *
 * Generator: Philox4x32-10, the counter-based generator of Salmon, Moraes,
 * Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11):
 * ten rounds of two 32x32->64-bit multiplies, with the key bumped by the
 * Weyl constants between rounds. Counter = (block index lo, block index hi,
 * stream, 0); key = (seed lo, seed hi). One block yields four 32-bit words.
 *
 * Normals: Box-Muller in double precision on pairs of words, each word mapped
 * to the open interval (0, 1) as (x + 0.5) / 2^32. Element i uses word i % 4
 * of block i / 4. The double result is scaled by `std`, rounded to float
 * (round-to-nearest-even, the C cast), and for bf16 rounded again from float
 * to bf16 by round-to-nearest-even on the bit pattern.
 *
 * Built with gcc -O2 -ffp-contract=off; OpenMP splits the element range only,
 * so the output does not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static inline void philox_round(uint32_t c[4], const uint32_t k[2]) {
    uint64_t p0 = (uint64_t)PHILOX_M0 * c[0];
    uint64_t p1 = (uint64_t)PHILOX_M1 * c[2];
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c[1] ^ k[0];
    uint32_t n2 = hi0 ^ c[3] ^ k[1];
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
}

void syn_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
    uint32_t c[4] = {ctr_in[0], ctr_in[1], ctr_in[2], ctr_in[3]};
    uint32_t k[2] = {key_in[0], key_in[1]};
    for (int r = 0; r < 10; ++r) {
        philox_round(c, k);
        k[0] += PHILOX_W0;
        k[1] += PHILOX_W1;
    }
    /* the tenth round's key bump is unused, as in the published algorithm */
    memcpy(out, c, sizeof(c));
}

static inline void block_words(uint64_t seed, uint32_t stream, uint64_t blk, uint32_t w[4]) {
    uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), stream, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    syn_philox4x32_10(ctr, key, w);
}

static inline double to_open01(uint32_t x) { return ((double)x + 0.5) * (1.0 / 4294967296.0); }

static inline void box_muller(uint32_t a, uint32_t b, double* z0, double* z1) {
    const double two_pi = 6.283185307179586476925286766559;
    double r = sqrt(-2.0 * log(to_open01(a)));
    double t = two_pi * to_open01(b);
    *z0 = r * cos(t);
    *z1 = r * sin(t);
}

static inline uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static inline void normals_of_block(uint64_t seed, uint32_t stream, uint64_t blk, double z[4]) {
    uint32_t w[4];
    block_words(seed, stream, blk, w);
    box_muller(w[0], w[1], &z[0], &z[1]);
    box_muller(w[2], w[3], &z[2], &z[3]);
}

/* out[i] = float(std * N_i) for element i in [first, first + n). */
void syn_normal_f32(uint64_t seed, uint32_t stream, int64_t first, int64_t n, double std_, float* out) {
    if (n <= 0) return;
    int64_t b0 = first / 4, b1 = (first + n + 3) / 4;
#pragma omp parallel for schedule(static)
    for (int64_t blk = b0; blk < b1; ++blk) {
        double z[4];
        normals_of_block(seed, stream, (uint64_t)blk, z);
        for (int s = 0; s < 4; ++s) {
            int64_t i = blk * 4 + s;
            if (i >= first && i < first + n) out[i - first] = (float)(std_ * z[s]);
        }
    }
}

/* out[i] = bf16(float(std * N_i)) as raw bits. */
void syn_normal_bf16(uint64_t seed, uint32_t stream, int64_t first, int64_t n, double std_, uint16_t* out) {
    if (n <= 0) return;
    int64_t b0 = first / 4, b1 = (first + n + 3) / 4;
#pragma omp parallel for schedule(static)
    for (int64_t blk = b0; blk < b1; ++blk) {
        double z[4];
        normals_of_block(seed, stream, (uint64_t)blk, z);
        for (int s = 0; s < 4; ++s) {
            int64_t i = blk * 4 + s;
            if (i >= first && i < first + n) out[i - first] = f32_to_bf16_rne((float)(std_ * z[s]));
        }
    }
}

/* Raw 32-bit words, element i = word i % 4 of block i / 4. */
void syn_u32(uint64_t seed, uint32_t stream, int64_t first, int64_t n, uint32_t* out) {
    if (n <= 0) return;
    int64_t b0 = first / 4, b1 = (first + n + 3) / 4;
#pragma omp parallel for schedule(static)
    for (int64_t blk = b0; blk < b1; ++blk) {
        uint32_t w[4];
        block_words(seed, stream, (uint64_t)blk, w);
        for (int s = 0; s < 4; ++s) {
            int64_t i = blk * 4 + s;
            if (i >= first && i < first + n) out[i - first] = w[s];
        }
    }
}
