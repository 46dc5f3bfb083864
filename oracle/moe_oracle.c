/*
 * moe_oracle.c -- plain fp64 CPU oracle for the group-quantized MoE FFN block.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library; it reads the canonical weight
 * record layout with its own decoding and computes everything in fp64 with
 * plain loops, in the order the definitions state.
 *
 * Sources (web pages about the Flash-MoE engine):
 *  [A2A]  "Flash-MoE란 무엇인가? 노트북에서 397B 파라미터 AI 모델 실행하기",
 *         a2a-mcp.org/blog/what-is-flash-moe-ko -- "Understanding MoE" section
 *         (4 of 512 routed experts + 1 shared per layer), "Key specs" list,
 *         deep dive 2 "FMA-optimized dequantization kernel" (the naive
 *         nibble*scale+bias form and its fma rearrangement), deep dive 3
 *         "Hand-tuned Metal compute shaders" (fused SwiGLU, two-pass RMSNorm,
 *         MoE combine + residual + sigmoid gating in one pass).
 *  [WIKI] "Flash-MoE — 순수 C/Metal로 M3 Max에서 397B MoE 모델 실행",
 *         jeongsk-2ndbrain.pages.dev -- "Target model" (hidden 4096, K=4 of 512
 *         plus one shared expert), technique 2 "FMA dequant kernel", technique
 *         3 "hand-written Metal kernels", "Per-layer pipeline" (CPU softmax +
 *         top-K between command buffers; CMD3 = expert forward + combine + norm).
 *  [GILLI] "flash-moe로 Apple Silicon에서 MoE 모델 추론하기", blog.gillilab.com
 *         -- section "Quantization / attention / cache / prefetching": group
 *         quantization keeps a scale and a zero point per group of 64 or 128
 *         weights.
 *
 * Readings where the pages leave a step open (each is also listed in the
 * design notes): codes are packed low bits first (q4: element c in byte c/2,
 * even c in the low nibble; q2: element c at bits 2*(c%4) of byte c/4); a
 * group is 64 consecutive elements along a row (the input dimension); scale and
 * bias are bf16 planes [R][C/G] that follow the codes of each matrix; softmax
 * is taken over all experts and the k selected probabilities are renormalised;
 * top-k ties go to the lower expert index and the output is in descending
 * logit order; the shared-expert gate is sigmoid(w_sg . x); the stack norm is a
 * unit-gain RMSNorm.
 *
 * Parity pins: every exported function is pinned by CPU tests against closed
 * forms, hand-derived fixtures, invariants or exact rational arithmetic.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <string.h>

/* Threads of the OpenMP loops over output rows (the timing harness runs the oracle at one
 * thread and at all cores; the arithmetic of each row does not depend on the count). */
void orc_set_num_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
int orc_max_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------------------------------- */
/* canonical record geometry                                                 */
/* ------------------------------------------------------------------------- */

static int64_t codes_bytes(int bits, int R, int C) { return (int64_t)R * C * bits / 8; }
static int64_t meta_count(int R, int C, int G) { return (int64_t)R * (C / G); }

/* bytes of one [R x C] matrix record: codes | scale bf16 | bias bf16 */
int64_t orc_matrix_bytes(int bits, int R, int C, int G) {
  return codes_bytes(bits, R, C) + 4 * meta_count(R, C, G);
}

/* bytes of one expert record: gate [I x H] | up [I x H] | down [H x I] */
int64_t orc_expert_bytes(int bits, int H, int I, int G) {
  return 2 * orc_matrix_bytes(bits, I, H, G) + orc_matrix_bytes(bits, H, I, G);
}

/* bf16 bit pattern -> value (bf16 is the top half of an IEEE single) */
static double bf16_value(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* integer code of element (r, c) */
static int code_at(int bits, int C, const uint8_t* codes, int r, int c) {
  if (bits == 4) {
    uint8_t byte = codes[(int64_t)r * (C / 2) + c / 2];
    return (c % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
  } else { /* bits == 2 */
    uint8_t byte = codes[(int64_t)r * (C / 4) + c / 4];
    return (byte >> (2 * (c % 4))) & 0x03;
  }
}

/*
 * O1 -- dequantized weight, the naive form of [A2A] deep dive 2 and [WIKI]
 * technique 2: weight = code * scale + bias, with scale and bias taken from
 * the element's group ([GILLI], group quantization).
 */
static double dequant_at(int bits, int R, int C, int G, const uint8_t* rec, int r, int c) {
  const uint8_t* codes = rec;
  const uint16_t* scale = (const uint16_t*)(rec + codes_bytes(bits, R, C));
  const uint16_t* bias = scale + meta_count(R, C, G);
  int64_t gi = (int64_t)r * (C / G) + c / G;
  double q = (double)code_at(bits, C, codes, r, c);
  return q * bf16_value(scale[gi]) + bf16_value(bias[gi]);
}

/* Full dequantized matrix W [R][C] (O1). */
void orc_dequant(int bits, int R, int C, int G, const uint8_t* rec, double* W) {
  for (int r = 0; r < R; ++r)
    for (int c = 0; c < C; ++c) W[(int64_t)r * C + c] = dequant_at(bits, R, C, G, rec, r, c);
}

/* y = deq(W) x : naive dequantize-then-dot ([A2A] deep dive 2, "before"). */
void orc_qmatvec(int bits, int R, int C, int G, const uint8_t* rec, const double* x, double* y) {
#pragma omp parallel for schedule(static)
  for (int r = 0; r < R; ++r) {
    double acc = 0.0;
    for (int c = 0; c < C; ++c) acc += dequant_at(bits, R, C, G, rec, r, c) * x[c];
    y[r] = acc;
  }
}

/*
 * O9 -- the rearranged form of [A2A] deep dive 2 / [WIKI] technique 2: with
 * scale*x and bias*x formed first, each element contributes one fused
 * multiply-add fma(code, scale*x, bias*x).  Used only to test that the
 * rearrangement is an identity.
 */
void orc_qmatvec_fma_form(int bits, int R, int C, int G, const uint8_t* rec, const double* x,
                          double* y) {
  const uint8_t* codes = rec;
  const uint16_t* scale = (const uint16_t*)(rec + codes_bytes(bits, R, C));
  const uint16_t* bias = scale + meta_count(R, C, G);
  for (int r = 0; r < R; ++r) {
    double acc = 0.0;
    for (int c = 0; c < C; ++c) {
      int64_t gi = (int64_t)r * (C / G) + c / G;
      double sx = bf16_value(scale[gi]) * x[c];
      double bx = bf16_value(bias[gi]) * x[c];
      acc += fma((double)code_at(bits, C, codes, r, c), sx, bx);
    }
    y[r] = acc;
  }
}

/*
 * O9 -- the same sum regrouped per quantization group: scale times the
 * code-weighted input sum plus bias times the plain input sum of the group.
 */
void orc_qmatvec_xsum_form(int bits, int R, int C, int G, const uint8_t* rec, const double* x,
                           double* y) {
  const uint8_t* codes = rec;
  const uint16_t* scale = (const uint16_t*)(rec + codes_bytes(bits, R, C));
  const uint16_t* bias = scale + meta_count(R, C, G);
  for (int r = 0; r < R; ++r) {
    double acc = 0.0;
    for (int g = 0; g < C / G; ++g) {
      double qx = 0.0, xs = 0.0;
      for (int c = g * G; c < (g + 1) * G; ++c) {
        qx += (double)code_at(bits, C, codes, r, c) * x[c];
        xs += x[c];
      }
      int64_t gi = (int64_t)r * (C / G) + g;
      acc += bf16_value(scale[gi]) * qx + bf16_value(bias[gi]) * xs;
    }
    y[r] = acc;
  }
}

/*
 * O4 -- one expert FFN with fused SwiGLU ([A2A] deep dive 3, [WIKI] technique
 * 3): g = W_gate x, u = W_up x, h = silu(g) * u with silu(g) = g / (1 + e^-g),
 * y = W_down h.  Any of g, u, h may be NULL.
 */
void orc_expert_ffn(int bits, int H, int I, int G, const uint8_t* expert, const double* x,
                    double* g_out, double* u_out, double* h_out, double* y) {
  int64_t mg = orc_matrix_bytes(bits, I, H, G);
  const uint8_t* gate = expert;
  const uint8_t* up = expert + mg;
  const uint8_t* down = expert + 2 * mg;
  double g[I], u[I], h[I]; /* I is small (<= a few thousand) */
  orc_qmatvec(bits, I, H, G, gate, x, g);
  orc_qmatvec(bits, I, H, G, up, x, u);
  for (int i = 0; i < I; ++i) h[i] = g[i] / (1.0 + exp(-g[i])) * u[i];
  orc_qmatvec(bits, H, I, G, down, h, y);
  if (g_out) memcpy(g_out, g, sizeof(double) * I);
  if (u_out) memcpy(u_out, u, sizeof(double) * I);
  if (h_out) memcpy(h_out, h, sizeof(double) * I);
}

/* O2 -- router logits l[e] = sum_c W_r[e][c] x[c] ([WIKI] per-layer pipeline, CMD2 routing). */
void orc_router_logits(int E, int H, const float* w_router, const double* x, double* logits) {
#pragma omp parallel for schedule(static)
  for (int e = 0; e < E; ++e) {
    double acc = 0.0;
    for (int c = 0; c < H; ++c) acc += (double)w_router[(int64_t)e * H + c] * x[c];
    logits[e] = acc;
  }
}

/* softmax over all E logits, with the maximum subtracted first; a NaN logit
 * gets probability 0 (it can never be selected, see orc_topk) */
void orc_softmax(int E, const double* logits, double* p) {
  double m = -INFINITY;
  for (int e = 0; e < E; ++e)
    if (logits[e] > m) m = logits[e];
  double s = 0.0;
  for (int e = 0; e < E; ++e) {
    p[e] = isnan(logits[e]) ? 0.0 : exp(logits[e] - m);
    s += p[e];
  }
  for (int e = 0; e < E; ++e) p[e] /= s;
}

/*
 * O3 -- top-k selection and renormalised weights ([WIKI] per-layer pipeline:
 * softmax + top-K on the CPU; [A2A] 4 routed experts per layer).  Selection
 * repeats "largest remaining logit"; on equal logits the lower index wins; NaN
 * logits are never selected (unselected slots get id -1, weight 0).  Weights
 * are the softmax probabilities of the selected experts divided by their sum.
 */
void orc_topk(int E, int k, const double* logits, int32_t* ids, double* weights) {
  double p[E];
  unsigned char taken[E];
  memset(taken, 0, (size_t)E);
  orc_softmax(E, logits, p);
  double total = 0.0;
  for (int j = 0; j < k; ++j) {
    int best = -1;
    for (int e = 0; e < E; ++e) {
      if (taken[e] || isnan(logits[e])) continue;
      if (best < 0 || logits[e] > logits[best]) best = e;
    }
    ids[j] = best;
    if (best >= 0) {
      taken[best] = 1;
      total += p[best];
    }
  }
  for (int j = 0; j < k; ++j) weights[j] = (ids[j] >= 0) ? p[ids[j]] / total : 0.0;
}

/* O5 -- shared-expert gate sigmoid(w_sg . x) ([A2A] deep dive 3: sigmoid gating). */
double orc_shared_gate(int H, const float* w_sg, const double* x) {
  double a = 0.0;
  for (int c = 0; c < H; ++c) a += (double)w_sg[c] * x[c];
  return 1.0 / (1.0 + exp(-a));
}

/*
 * O6 -- combine + residual ([A2A] deep dive 3, [WIKI] technique 3):
 * out = residual + sum_j w_j y_j + sg * y_shared, where y holds k routed rows
 * followed by the shared row.
 */
void orc_combine(int H, int k, const double* residual, const double* y, const double* w,
                 double sg, double* out) {
  for (int c = 0; c < H; ++c) {
    double acc = residual[c];
    for (int j = 0; j < k; ++j) acc += w[j] * y[(int64_t)j * H + c];
    acc += sg * y[(int64_t)k * H + c];
    out[c] = acc;
  }
}

/*
 * O7 -- RMSNorm in two passes ([A2A] deep dive 3, [WIKI] technique 3): first
 * the mean of squares, then x / sqrt(mean + eps); unit gain.
 */
void orc_rmsnorm(int H, double eps, const double* x, double* out) {
  double ss = 0.0;
  for (int c = 0; c < H; ++c) ss += x[c] * x[c];
  double inv = 1.0 / sqrt(ss / H + eps);
  for (int c = 0; c < H; ++c) out[c] = x[c] * inv;
}
