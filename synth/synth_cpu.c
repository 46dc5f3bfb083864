/*
 * synth_cpu.c -- host side of the seeded synthetic-input generator.
 * The definitions of every draw live in synth.h; this file only loops.
 * Built with gcc -O2 -fopenmp -ffp-contract=off.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "synth.h"

/* Fill one [R x C] matrix record: codes | scale | bias. */
void synth_fill_matrix(uint8_t* out, uint64_t seed, int layer, int slot, int codes_tensor,
                       int scale_tensor, int bits, int R, int C, int G, double lo, double hi,
                       double zp) {
  uint64_t ncode = synth_codes_bytes(bits, R, C);
  uint64_t nmeta = synth_meta_count(R, C, G);
  uint64_t kc = synth_key(seed, (uint64_t)layer, (uint64_t)slot, (uint64_t)codes_tensor);
  uint64_t ks = synth_key(seed, (uint64_t)layer, (uint64_t)slot, (uint64_t)scale_tensor);
  uint64_t nwords = ncode / 8;
#pragma omp parallel for schedule(static)
  for (int64_t w = 0; w < (int64_t)nwords; ++w) {
    uint64_t d = synth_draw(kc, (uint64_t)w);
    memcpy(out + 8 * w, &d, 8); /* little-endian: byte j%8 of draw j/8 */
  }
  for (uint64_t j = nwords * 8; j < ncode; ++j) out[j] = synth_code_byte(kc, j);
  uint16_t* sc = (uint16_t*)(out + ncode);
  uint16_t* bi = sc + nmeta;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)nmeta; ++i) {
    uint16_t s = synth_scale_bf16(synth_draw(ks, (uint64_t)i), lo, hi);
    sc[i] = s;
    bi[i] = synth_bias_bf16(s, zp);
  }
}

/* Fill one expert record: gate [I x H], up [I x H], down [H x I]. */
void synth_fill_expert(uint8_t* out, uint64_t seed, int layer, int slot, int bits, int H, int I,
                       int G, double lo, double hi, double zp) {
  uint64_t mg = synth_matrix_bytes(bits, I, H, G);
  synth_fill_matrix(out, seed, layer, slot, SYNTH_T_GATE_CODES, SYNTH_T_GATE_SCALE, bits, I, H, G,
                    lo, hi, zp);
  synth_fill_matrix(out + mg, seed, layer, slot, SYNTH_T_UP_CODES, SYNTH_T_UP_SCALE, bits, I, H, G,
                    lo, hi, zp);
  synth_fill_matrix(out + 2 * mg, seed, layer, slot, SYNTH_T_DOWN_CODES, SYNTH_T_DOWN_SCALE, bits,
                    H, I, G, lo, hi, zp);
}

/* n fp32 draws of N(0, sigma^2): Box-Muller on draws 2i, 2i+1 of the stream. */
void synth_fill_normal(float* out, uint64_t n, uint64_t seed, int layer, int slot, int tensor,
                       double sigma) {
  const double two_pi = 6.283185307179586476925286766559;
  uint64_t k = synth_key(seed, (uint64_t)layer, (uint64_t)slot, (uint64_t)tensor);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < (int64_t)n; ++i) {
    uint64_t d1 = synth_draw(k, 2 * (uint64_t)i);
    uint64_t d2 = synth_draw(k, 2 * (uint64_t)i + 1);
    double u1 = ((double)(d1 >> 11) + 1.0) * (1.0 / 9007199254740992.0); /* (0, 1] */
    double u2 = (double)(d2 >> 11) * (1.0 / 9007199254740992.0);         /* [0, 1) */
    double r = sqrt(-2.0 * log(u1));
    double z = r * cos(two_pi * u2);
    out[i] = (float)(z * sigma);
  }
}

uint64_t synth_expert_nbytes(int bits, int H, int I, int G) {
  return synth_expert_bytes(bits, H, I, G);
}

uint64_t synth_key_export(uint64_t seed, uint64_t layer, uint64_t slot, uint64_t tensor) {
  return synth_key(seed, layer, slot, tensor);
}

uint64_t synth_draw_export(uint64_t key, uint64_t i) { return synth_draw(key, i); }

uint16_t synth_f64_to_bf16_export(double v) { return synth_f64_to_bf16(v); }
