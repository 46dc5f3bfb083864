/*
 * synth.h -- seeded synthetic-input generator (test and benchmark input only).
 *
 * This header defines how every synthetic tensor of the benchmark workloads is
 * drawn: quantization codes, bf16 group scales and biases, and the fp32 normal
 * draws for activations and router weights.  It contains none of the MoE
 * arithmetic (no dequantization, no products, no routing); it only produces
 * bytes.  The same definitions are compiled for the host (synth_cpu.c) and for
 * the device fill kernels (synth_gpu.hip), so both sides write identical bytes.
 *
 * Generator: SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014), used counter-style: the i-th output of the
 * stream whose state starts at key k is mix64(k + (i + 1) * GAMMA).  A stream
 * key is derived from (seed, layer, slot, tensor) by chained mixing.
 *
 * Record layout written by the fill routines (one expert "slot"):
 *   gate [I x H], up [I x H], down [H x I]; each matrix [R x C] is
 *   codes u8[R][C*bits/8] | scale bf16[R][C/G] | bias bf16[R][C/G].
 *   q4: element c of a row sits in byte c/2, even c in the low nibble.
 *   q2: element c sits in byte c/4 at bits 2*(c%4).
 * Codes: every code byte is one byte of a 64-bit draw (byte j of a matrix is
 *   byte j%8 of draw j/8), so every nibble / 2-bit field is uniform.
 * Scales: draw d -> u = (d >> 11) * 2^-53 in [0,1); s = lo + (hi - lo) * u in
 *   fp64 without contraction, rounded to bf16 (round to nearest even).
 * Biases: b = -zp * s in fp64, rounded to bf16 (nearest even): exact for q4's zero point 8;
 *   q2's 1.5 puts the codes 0..3 symmetric about zero (a q2 zero point of 2 gives every
 *   weight a mean of -s/2, which makes stacked layers saturate the SwiGLU), and -1.5 s can
 *   round.
 * Normals: Box-Muller in fp64 from draws 2i and 2i+1, times sigma, rounded to
 *   fp32.  Normals are produced on the host only (libm differs between host and
 *   device), and uploaded.
 */
#ifndef SYNTH_H
#define SYNTH_H

#include <stdint.h>

#if defined(__HIPCC__)
#define SYNTH_FN __host__ __device__ static inline
#else
#define SYNTH_FN static inline
#endif

#define SYNTH_GAMMA 0x9E3779B97F4A7C15ULL

/* tensor identifiers inside a stream key */
enum {
  SYNTH_T_GATE_CODES = 0,
  SYNTH_T_GATE_SCALE = 1,
  SYNTH_T_UP_CODES = 2,
  SYNTH_T_UP_SCALE = 3,
  SYNTH_T_DOWN_CODES = 4,
  SYNTH_T_DOWN_SCALE = 5,
  SYNTH_T_ROUTER = 16,
  SYNTH_T_SHARED_GATE = 17,
  SYNTH_T_X = 32
};

SYNTH_FN uint64_t synth_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

SYNTH_FN uint64_t synth_key(uint64_t seed, uint64_t layer, uint64_t slot, uint64_t tensor) {
  uint64_t k = synth_mix64(seed + SYNTH_GAMMA);
  k = synth_mix64(k + (layer + 1) * SYNTH_GAMMA);
  k = synth_mix64(k + (slot + 1) * SYNTH_GAMMA);
  k = synth_mix64(k + (tensor + 1) * SYNTH_GAMMA);
  return k;
}

/* i-th output of the SplitMix64 stream started at key */
SYNTH_FN uint64_t synth_draw(uint64_t key, uint64_t i) {
  return synth_mix64(key + (i + 1) * SYNTH_GAMMA);
}

/* fp64 -> bf16 bits, round to nearest even; finite normal inputs only */
SYNTH_FN uint16_t synth_f64_to_bf16(double v) {
  union { double d; uint64_t u; } cv;
  cv.d = v;
  uint64_t bits = cv.u;
  uint64_t sign = bits >> 63;
  int64_t exp = (int64_t)((bits >> 52) & 0x7FF) - 1023 + 127;
  uint64_t mant = bits & 0xFFFFFFFFFFFFFULL;      /* 52 bits */
  uint64_t keep = mant >> 45;                       /* top 7 bits */
  uint64_t rest = mant & ((1ULL << 45) - 1);
  uint64_t half = 1ULL << 44;
  if (rest > half || (rest == half && (keep & 1))) {
    keep += 1;
    if (keep == 128) { keep = 0; exp += 1; }
  }
  return (uint16_t)((sign << 15) | ((uint64_t)exp << 7) | keep);
}

/* bf16 bits -> fp32 (exact) */
SYNTH_FN float synth_bf16_to_f32(uint16_t b) {
  union { uint32_t u; float f; } cv;
  cv.u = ((uint32_t)b) << 16;
  return cv.f;
}

SYNTH_FN uint16_t synth_f32_to_bf16_exact(float f) {
  union { float f; uint32_t u; } cv;
  cv.f = f;
  return (uint16_t)(cv.u >> 16);
}

/* scale draw: s = bf16(lo + (hi - lo) * u) */
SYNTH_FN uint16_t synth_scale_bf16(uint64_t draw, double lo, double hi) {
#if defined(__clang__)
#pragma clang fp contract(off)
#endif
  double u = (double)(draw >> 11) * (1.0 / 9007199254740992.0);
  double w = hi - lo;
  double t = w * u;
  double s = lo + t;
  return synth_f64_to_bf16(s);
}

/* bias = bf16(-zp * scale), rounded to nearest even: exact for q4's power-of-two zero point
   (8); q2's 1.5 centres the four codes, and -1.5 s can need one bit more than bf16 holds */
SYNTH_FN uint16_t synth_bias_bf16(uint16_t scale_bits, double zp) {
  double s = (double)synth_bf16_to_f32(scale_bits);
  return synth_f64_to_bf16(-(zp * s));
}

/* code byte j of a matrix stream */
SYNTH_FN uint8_t synth_code_byte(uint64_t key, uint64_t j) {
  return (uint8_t)(synth_draw(key, j >> 3) >> (8 * (j & 7)));
}

/* ---- record geometry (bytes) ---- */
SYNTH_FN uint64_t synth_codes_bytes(int bits, int R, int C) { return (uint64_t)R * C * bits / 8; }
SYNTH_FN uint64_t synth_meta_count(int R, int C, int G) { return (uint64_t)R * (C / G); }
SYNTH_FN uint64_t synth_matrix_bytes(int bits, int R, int C, int G) {
  return synth_codes_bytes(bits, R, C) + 2 * 2 * synth_meta_count(R, C, G);
}
SYNTH_FN uint64_t synth_expert_bytes(int bits, int H, int I, int G) {
  return 2 * synth_matrix_bytes(bits, I, H, G) + synth_matrix_bytes(bits, H, I, G);
}

#endif /* SYNTH_H */
