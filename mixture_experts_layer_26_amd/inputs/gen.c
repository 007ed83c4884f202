/*
 * Seeded, counter-based synthetic input generator.
 *
 * Shared by the HIP path's tests/bench and by the CPU oracle's tests: it only
 * draws numbers (normal and uniform variates, rounded to the storage type) and
 * holds none of the layer's arithmetic.
 *
 * Bits: Philox4x32-10, as published by Salmon, Moraes, Dror and Shaw,
 * "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11).  The 128-bit counter
 * is (block_lo, block_hi, tensor_id, 0) and the 64-bit key is the seed, so
 * element i of tensor `tid` depends only on (seed, tid, i): any slice (one
 * expert's weights, one token's row) can be regenerated on its own, and the
 * result does not depend on the thread count.
 *
 * Normals: the Box-Muller transform (Box and Muller, 1958) on the pairs
 * (r0, r1) and (r2, r3) of one Philox block, giving 4 variates per block.
 * Uniforms in (0,1) are (r + 0.5) * 2^-32.
 */
#define _GNU_SOURCE
#include <math.h>
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

void gen_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int r = 0; r < 10; ++r) {
    uint64_t p0 = (uint64_t)PHILOX_M0 * c0;
    uint64_t p1 = (uint64_t)PHILOX_M1 * c2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0; c1 = lo1; c2 = n2; c3 = lo0;
    k0 += PHILOX_W0; k1 += PHILOX_W1;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

static inline void block_bits(uint64_t seed, uint32_t tid, uint64_t blk, uint32_t r[4]) {
  uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), tid, 0u};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  gen_philox4x32_10(ctr, key, r);
}

static inline double unit_open(uint32_t r) { return ((double)r + 0.5) * 0x1p-32; }

/* the four standard normals of Philox block `blk` */
static inline void block_normals(uint64_t seed, uint32_t tid, uint64_t blk, double z[4]) {
  uint32_t r[4];
  block_bits(seed, tid, blk, r);
  const double two_pi = 6.283185307179586476925286766559;
  double rad0 = sqrt(-2.0 * log(unit_open(r[0])));
  double ang0 = two_pi * unit_open(r[1]);
  double rad1 = sqrt(-2.0 * log(unit_open(r[2])));
  double ang1 = two_pi * unit_open(r[3]);
  double s0, c0, s1, c1;
  sincos(ang0, &s0, &c0);
  sincos(ang1, &s1, &c1);
  z[0] = rad0 * c0;
  z[1] = rad0 * s0;
  z[2] = rad1 * c1;
  z[3] = rad1 * s1;
}

/* fp32 -> bf16 bits, round to nearest even (inputs are finite) */
static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* out[j] = fl32(stddev * z(start + j)), j < n */
void gen_normal_f32(uint64_t seed, uint32_t tid, uint64_t start, uint64_t n, double stddev, float* out) {
  const int64_t first = (int64_t)(start >> 2), last = (int64_t)((start + n + 3) >> 2);
#pragma omp parallel for schedule(static) if (n > 65536)
  for (int64_t blk = first; blk < last; ++blk) {
    double z[4];
    block_normals(seed, tid, (uint64_t)blk, z);
    for (int q = 0; q < 4; ++q) {
      uint64_t i = ((uint64_t)blk << 2) + (uint64_t)q;
      if (i >= start && i < start + n) out[i - start] = (float)(stddev * z[q]);
    }
  }
}

/* out[j] = bf16_rne(fl32(stddev * z(start + j))) */
void gen_normal_bf16(uint64_t seed, uint32_t tid, uint64_t start, uint64_t n, double stddev, uint16_t* out) {
  const int64_t first = (int64_t)(start >> 2), last = (int64_t)((start + n + 3) >> 2);
#pragma omp parallel for schedule(static) if (n > 65536)
  for (int64_t blk = first; blk < last; ++blk) {
    double z[4];
    block_normals(seed, tid, (uint64_t)blk, z);
    for (int q = 0; q < 4; ++q) {
      uint64_t i = ((uint64_t)blk << 2) + (uint64_t)q;
      if (i >= start && i < start + n) out[i - start] = f32_to_bf16_rne((float)(stddev * z[q]));
    }
  }
}

/* out[j] = fl32(lo + (hi - lo) * U(start + j)), U from the first word of each block */
void gen_uniform_f32(uint64_t seed, uint32_t tid, uint64_t start, uint64_t n, double lo, double hi, float* out) {
#pragma omp parallel for schedule(static) if (n > 65536)
  for (int64_t j = 0; j < (int64_t)n; ++j) {
    uint32_t r[4];
    block_bits(seed, tid, start + (uint64_t)j, r);
    out[j] = (float)(lo + (hi - lo) * unit_open(r[0]));
  }
}
