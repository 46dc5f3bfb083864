// moe_device.h -- device building blocks of libmoe (gfx950, wave64).
//
// Dequant matvec scheme.  A weight row is cut into 16-byte chunks of codes
// (32 q4 codes = half a group of 64, or 64 q2 codes = one group).  Lane l of a
// wave always owns the same chunk positions of every row it visits, so the
// inputs x of those positions live in registers for the whole kernel, together
// with their per-chunk sum X.  Each chunk then contributes
//     scale * sum(code_i * x_i) + bias * X
// which equals sum((code_i * scale + bias) * x_i), the naive dequant-then-dot
// (a2a-mcp.org "What is Flash-MoE", deep dive 2: the fma rearrangement is the
// same identity; here scale and bias are applied once per chunk instead of
// once per element).  Per-row partials are reduced across the lanes sharing
// the row with cross-lane adds.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;
constexpr int kGroup = 64;

__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Non-temporal 16-byte load: weights are streamed once per token, so they should not
// displace reusable lines (activations, routing tables) from the caches.
__device__ __forceinline__ uint4 ld_nt_u4(const void* p) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ float4 ld_nt_f4(const float* p) {
  typedef float v4f __attribute__((ext_vector_type(4)));
  const v4f v = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
  return make_float4(v[0], v[1], v[2], v[3]);
}

// bytes of one [R x C] matrix record (codes | scale bf16 | bias bf16), group 64
template <int BITS>
__host__ __device__ constexpr size_t matrix_rec_bytes(int R, int C) {
  return (size_t)R * C * BITS / 8 + 4 * (size_t)R * (C / kGroup);
}

// Geometry of one quantized row of C inputs for BITS-bit codes.
template <int BITS, int C>
struct Geo {
  static constexpr int kCodesPerChunk = 128 / BITS;               // codes in 16 bytes
  static constexpr int kChunksPerRow = C / kCodesPerChunk;
  static constexpr int kLanesPerRow = kChunksPerRow >= kWave ? kWave : kChunksPerRow;
  static constexpr int kRowsPerWave = kWave / kLanesPerRow;       // rows covered by one pass
  static constexpr int kPasses = kChunksPerRow / kLanesPerRow;    // chunks per lane per row
  static constexpr int kXPerLane = kPasses * kCodesPerChunk;      // inputs held per lane
  static constexpr int kRowBytes = C * BITS / 8;
  static constexpr int kGroupsPerRow = C / kGroup;
  static constexpr int kChunksPerGroup = kGroup / kCodesPerChunk;  // 2 (q4) or 1 (q2)
  static_assert((kChunksPerRow & (kChunksPerRow - 1)) == 0, "chunks per row must be 2^n");
  static_assert(kChunksPerRow % kLanesPerRow == 0, "");
};

// Code bytes to floats.  Every code sits alone in a byte after masking, and a byte b in
// 0..15 read as an OCP FP8 E4M3 value is exactly b * 2^-9 (E4M3 subnormals and its first
// binade are both spaced 2^-9), so one v_cvt_pk_f32_fp8 turns two codes into two floats.
// The 2^-9 is folded into the chunk's scale (kCodeUnit).
constexpr float kCodeUnit = 512.f;

template <bool HI_WORD>
__device__ __forceinline__ void codes2(uint32_t bytes, float& a, float& b) {
  const auto v = __builtin_amdgcn_cvt_pk_f32_fp8((int)bytes, HI_WORD);
  a = v[0];
  b = v[1];
}

// sum(code_i * x_i) / 512 over one 16-byte chunk of q4 codes; x in natural element order.
// Element 2j sits in the low nibble of byte j, 2j+1 in the high nibble.
__device__ __forceinline__ float dot_chunk_q4(const uint4 c, const float* __restrict__ x) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t lo = w[d] & 0x0F0F0F0Fu;          // bytes: elements 8d + 0, 2, 4, 6
    const uint32_t hi = (w[d] >> 4) & 0x0F0F0F0Fu;   // bytes: elements 8d + 1, 3, 5, 7
    const float* xd = x + 8 * d;
    float q0, q2, q4, q6, q1, q3, q5, q7;
    codes2<false>(lo, q0, q2);
    codes2<true>(lo, q4, q6);
    codes2<false>(hi, q1, q3);
    codes2<true>(hi, q5, q7);
    acc0 = fmaf(q0, xd[0], acc0);
    acc1 = fmaf(q1, xd[1], acc1);
    acc0 = fmaf(q2, xd[2], acc0);
    acc1 = fmaf(q3, xd[3], acc1);
    acc0 = fmaf(q4, xd[4], acc0);
    acc1 = fmaf(q5, xd[5], acc1);
    acc0 = fmaf(q6, xd[6], acc0);
    acc1 = fmaf(q7, xd[7], acc1);
  }
  return acc0 + acc1;
}

// sum(code_i * x_i) / 512 over one 16-byte chunk of q2 codes; element c at bits 2*(c%4)
// of byte c/4.
__device__ __forceinline__ float dot_chunk_q2(const uint4 c, const float* __restrict__ x) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const float* xd = x + 16 * d;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t f = (w[d] >> (2 * m)) & 0x03030303u;  // bytes: elements 16d + 4j + m
      float q0, q1, q2, q3;
      codes2<false>(f, q0, q1);  // j = 0, 1
      codes2<true>(f, q2, q3);   // j = 2, 3
      acc0 = fmaf(q0, xd[m], acc0);
      acc1 = fmaf(q1, xd[4 + m], acc1);
      acc0 = fmaf(q2, xd[8 + m], acc0);
      acc1 = fmaf(q3, xd[12 + m], acc1);
    }
  }
  return acc0 + acc1;
}

template <int BITS>
__device__ __forceinline__ float dot_chunk(const uint4 c, const float* __restrict__ x) {
  if constexpr (BITS == 4)
    return dot_chunk_q4(c, x);
  else
    return dot_chunk_q2(c, x);
}

// ---- cross-lane reductions on DPP (VALU data-parallel primitives, no LDS traffic) ----
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;  // row_ror:4
constexpr int kDppRowRor8 = 0x128;  // row_ror:8

// every lane of each 16-lane row receives the row's sum
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_f<kDppQuadXor1>(v);
  v += dpp_f<kDppQuadXor2>(v);
  v += dpp_f<kDppRowRor4>(v);
  v += dpp_f<kDppRowRor8>(v);
  return v;
}

__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Sum over aligned segments of W lanes (W in {16, 32, 64}, or a smaller power of two); every
// lane gets its segment's sum.  The order of additions is fixed, so every wave that reduces
// the same values gets the same bits.
template <int W>
__device__ __forceinline__ float seg_sum(float v) {
  if constexpr (W >= 16) {
    v = row_sum16(v);
    if constexpr (W == 16) {
      return v;
    } else if constexpr (W == 32) {
      const float a = lane_f(v, 0) + lane_f(v, 16);
      const float b = lane_f(v, 32) + lane_f(v, 48);
      return (threadIdx.x & 32) ? b : a;
    } else {
      return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
    }
  } else {
#pragma unroll
    for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
  }
}

// ---- inputs as integer digit planes: exact q4 products on v_dot8_i32_i4 ----
// A group of 64 inputs is held in fixed point with NPL signed hex digits: X = rint(x 2^(B - E)),
// B = 4 NPL - 2, with 2^E above the group's largest magnitude; the digits are the hex digits of
// X + 0x88..8 (NPL eights), each minus 8.  Digit plane k of 8 consecutive inputs packs their
// digit k in one dword, input i in nibble i: the order in which v_dot8_i32_i4 pairs it with 8
// packed q4 codes.  A code c enters as the signed nibble c ^ 8 = c - 8, so
// sum c x = 2^(E - B) sum (c - 8) X + 8 sum x, exact in integers and rounded once; X is within 1/2
// of x 2^(B - E), i.e. 2^-(B + 1) of the group maximum (2^-27 with seven planes, 2^-19 with five).
typedef unsigned u32v4 __attribute__((ext_vector_type(4)));
constexpr int kXPlanes = 7;

// eight values below 2^28 in, their seven hex-digit planes out (an 8 x 8 transpose of 4-bit
// elements; row 7 comes out zero)
__device__ __forceinline__ void nibble_transpose8(uint32_t (&r)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t t = ((r[i] >> 16) ^ r[i + 4]) & 0x0000FFFFu;
    r[i + 4] ^= t;
    r[i] ^= t << 16;
  }
#pragma unroll
  for (int i = 0; i < 8; i += (i & 1) ? 3 : 1) {  // pairs (0,2) (1,3) (4,6) (5,7)
    const uint32_t t = ((r[i] >> 8) ^ r[i + 2]) & 0x00FF00FFu;
    r[i + 2] ^= t;
    r[i] ^= t << 8;
  }
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const uint32_t t = ((r[i] >> 4) ^ r[i + 1]) & 0x0F0F0F0Fu;
    r[i + 1] ^= t;
    r[i] ^= t << 4;
  }
}

// Digit planes of one unit of 16 inputs v held by one lane; the four units of a 64-input group
// must sit in one lane quad (the group maximum is taken across it).  pl[k] holds digit plane k
// as two dwords: inputs 0..7 and 8..15, or with EVEN_ODD the even inputs and the odd ones (the
// order of the q2 product).  Returns the unit's input sum and the group's digit unit 2^(E - B).
template <bool EVEN_ODD, int NPL = kXPlanes>
__device__ __forceinline__ void digit_unit16(const float (&v)[16], uint2 (&pl)[NPL], float& sum,
                                             float& unit) {
  static_assert(NPL >= 2 && NPL <= 7, "");
  constexpr uint32_t kOff = 0x88888888u >> (4 * (8 - NPL));  // NPL hex eights
  float m = 0.f;
  sum = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    m = fmaxf(m, fabsf(v[i]));
    sum += v[i];
  }
  m = fmaxf(m, dpp_f<kDppQuadXor1>(m));
  m = fmaxf(m, dpp_f<kDppQuadXor2>(m));
  // biased exponent e of the group maximum: 2^(e - 126) > max; scale 2^(B + 126 - e)
  const int e = min(max((int)(__float_as_uint(m) >> 23), 26), 254);
  const float scale = __uint_as_float((uint32_t)(4 * NPL + 251 - e) << 23);
  unit = __uint_as_float((uint32_t)(e + 3 - 4 * NPL) << 23);
  uint32_t r[2][8];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t d = (uint32_t)((int)rintf(v[i] * scale) + (int)kOff);
    if constexpr (EVEN_ODD)
      r[i & 1][i >> 1] = d;
    else
      r[i >> 3][i & 7] = d;
  }
  nibble_transpose8(r[0]);
  nibble_transpose8(r[1]);
#pragma unroll
  for (int k = 0; k < NPL; ++k) pl[k] = make_uint2(r[0][k] ^ 0x88888888u, r[1][k] ^ 0x88888888u);
}

// sum of c x over one 16-byte chunk of q4 codes (32 codes) against the digit planes xd of its
// inputs (plane dword d: inputs 8d .. 8d + 7), their sum xsum and digit unit
template <int NPL = kXPlanes>
__device__ __forceinline__ float dot_chunk_q4_int(const u32v4 q, const uint4 (&xd)[NPL],
                                                  float xsum, float unit) {
  int p[NPL] = {};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int c = (int)(q[d] ^ 0x88888888u);
#pragma unroll
    for (int k = 0; k < NPL; ++k) {
      const uint4 pl = xd[k];
      const int xw = (int)(d == 0 ? pl.x : d == 1 ? pl.y : d == 2 ? pl.z : pl.w);
      p[k] = __builtin_amdgcn_sdot8(c, xw, p[k], false);
    }
  }
  // |p[k]| <= 32 * 8 * 8: the four low planes fit an int exactly, the (up to three) high ones too
  static_assert(NPL >= 5 && NPL <= 7, "");
  const int lo = p[0] + (p[1] << 4) + (p[2] << 8) + (p[3] << 12);
  int hi = p[4];
  if constexpr (NPL > 5) hi += p[5] << 4;
  if constexpr (NPL > 6) hi += p[6] << 8;
  return unit * fmaf(65536.f, (float)hi, (float)lo) + 8.f * xsum;
}

// Per-lane view of one quantized matrix row set: which chunk positions the lane owns.
template <int BITS, int C>
struct LaneRow {
  using G = Geo<BITS, C>;
  int sub;                       // row within the wave's pass
  int chunk[G::kPasses];         // chunk index within the row, per pass
  float x[G::kXPerLane];         // inputs of the owned chunks
  float xsum[G::kPasses];        // per-chunk input sums

  __device__ __forceinline__ void set_lane(int lane) {
    sub = lane / G::kLanesPerRow;
#pragma unroll
    for (int p = 0; p < G::kPasses; ++p) chunk[p] = (lane % G::kLanesPerRow) + G::kLanesPerRow * p;
  }

  // load the lane's inputs (no arithmetic yet); chunk c's inputs start at xin + c * stride
  __device__ __forceinline__ void load_x(const float* __restrict__ xin,
                                         int stride = G::kCodesPerChunk) {
#pragma unroll
    for (int p = 0; p < G::kPasses; ++p) {
      const float4* src = reinterpret_cast<const float4*>(xin + chunk[p] * stride);
#pragma unroll
      for (int v = 0; v < G::kCodesPerChunk / 4; ++v) {
        const float4 t = src[v];
        float* d = x + p * G::kCodesPerChunk + 4 * v;
        d[0] = t.x;
        d[1] = t.y;
        d[2] = t.z;
        d[3] = t.w;
      }
    }
  }

  // per-chunk input sums
  __device__ __forceinline__ void finish() {
#pragma unroll
    for (int p = 0; p < G::kPasses; ++p) {
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < G::kCodesPerChunk; ++c) s += x[p * G::kCodesPerChunk + c];
      xsum[p] = s;
    }
  }

  __device__ __forceinline__ void init(int lane, const float* __restrict__ xin) {
    set_lane(lane);
    load_x(xin);
    finish();
  }
};

// Raw loads of one row's owned chunks: codes + the chunk's group scale and bias.
template <int BITS, int C>
struct RowLoad {
  using G = Geo<BITS, C>;
  uint4 q[G::kPasses];
  uint16_t s[G::kPasses];
  uint16_t b[G::kPasses];

  // rec: matrix record base (codes | scale | bias), R rows
  __device__ __forceinline__ void load(const uint8_t* __restrict__ rec, int R, int row,
                                       const LaneRow<BITS, C>& lr) {
    const uint8_t* codes = rec + (size_t)row * G::kRowBytes;
    const uint16_t* scale = reinterpret_cast<const uint16_t*>(rec + (size_t)R * G::kRowBytes);
    const uint16_t* bias = scale + (size_t)R * G::kGroupsPerRow;
#pragma unroll
    for (int p = 0; p < G::kPasses; ++p) {
      q[p] = ld_nt_u4(codes + lr.chunk[p] * 16);
      const int gi = row * G::kGroupsPerRow + lr.chunk[p] / G::kChunksPerGroup;
      s[p] = __builtin_nontemporal_load(scale + gi);
      b[p] = __builtin_nontemporal_load(bias + gi);
    }
  }

  // pass p's term of this lane's partial: inputs xp of the pass's chunk, their sum xsum
  __device__ __forceinline__ float term(int p, const float* __restrict__ xp, float xsum) const {
    const float qx = dot_chunk<BITS>(q[p], xp);
    return (bf16f(s[p]) * kCodeUnit) * qx + bf16f(b[p]) * xsum;
  }

  // 32-input records per chunk in term_int: one for q4, two for q2 (64 codes)
  static constexpr int kRecs = G::kCodesPerChunk / 32;

  // Pass p's term from the digit planes of the pass's chunk: record h covers inputs 32 h ..
  // 32 h + 31 of the chunk (q2: with the even and odd inputs of each 16 in that order), with its
  // input sum and digit unit.  A q2 word of 16 codes masked with 0x33333333 leaves the even codes
  // as nibbles, shifted right by 2 first the odd ones, so q2 takes the q4 product.
  template <int NPL>
  __device__ __forceinline__ float term_int(int p, const uint4 (&xd)[kRecs][NPL],
                                            const float (&xsum)[kRecs],
                                            const float (&unit)[kRecs]) const {
    float qx = 0.f, xs = 0.f;
    if constexpr (BITS == 4) {
      const u32v4 c = {q[p].x, q[p].y, q[p].z, q[p].w};
      qx = dot_chunk_q4_int<NPL>(c, xd[0], xsum[0], unit[0]);
      xs = xsum[0];
    } else {
      const uint32_t w[4] = {q[p].x, q[p].y, q[p].z, q[p].w};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32v4 c = {w[2 * h] & 0x33333333u, (w[2 * h] >> 2) & 0x33333333u,
                         w[2 * h + 1] & 0x33333333u, (w[2 * h + 1] >> 2) & 0x33333333u};
        qx += dot_chunk_q4_int<NPL>(c, xd[h], xsum[h], unit[h]);
      }
      xs = xsum[0] + xsum[1];
    }
    return bf16f(s[p]) * qx + bf16f(b[p]) * xs;
  }

  // this lane's partial of the row dot product
  __device__ __forceinline__ float partial(const LaneRow<BITS, C>& lr) const {
    float acc = 0.f;
#pragma unroll
    for (int p = 0; p < G::kPasses; ++p) acc += term(p, lr.x + p * G::kCodesPerChunk, lr.xsum[p]);
    return acc;
  }
};

// One-wave top-k over E <= 1024 logits (ties to the lower index, NaN never chosen),
// renormalised softmax weights over the selected.  Every lane returns the same values in
// ids/vals/w (kMaxTopK entries; entries >= k are left untouched).  ids[j] = -1 and w[j] = 0
// when fewer than j+1 logits are selectable.
//
// Each candidate is a 64-bit key: the logit mapped to an order-preserving unsigned integer
// in the high word and the complement of its index in the low word, so "larger key" means
// "larger logit, then lower index".  Key 0 marks "nothing".  A round takes every lane's
// best remaining key, reduces it across the wave (DPP within rows, readlane across rows),
// and the owning lane marks the winner taken.
constexpr int kMaxTopK = 8;

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) {
  uint32_t lo = (uint32_t)k, hi = (uint32_t)(k >> 32);
#define MOE_MAX_STEP(CTRL)                                              \
  {                                                                     \
    const uint32_t olo = dpp_u<CTRL>(lo), ohi = dpp_u<CTRL>(hi);        \
    const uint64_t o = ((uint64_t)ohi << 32) | olo;                     \
    const uint64_t m = ((uint64_t)hi << 32) | lo;                       \
    if (o > m) { lo = olo; hi = ohi; }                                  \
  }
  MOE_MAX_STEP(kDppQuadXor1)
  MOE_MAX_STEP(kDppQuadXor2)
  MOE_MAX_STEP(kDppRowRor4)
  MOE_MAX_STEP(kDppRowRor8)
#undef MOE_MAX_STEP
  uint64_t best = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint64_t c = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)hi, 16 * r) << 32) |
                       (uint32_t)__builtin_amdgcn_readlane((int)lo, 16 * r);
    best = c > best ? c : best;
  }
  return best;
}

// kPer = logits per lane (E <= 64 * kPer).  All loads are issued before any is used.
template <int kPer>
__device__ __forceinline__ void wave_topk_n(const float* __restrict__ logits, int E, int k,
                                            int* ids, float* vals, float* w) {
  const int lane = threadIdx.x & (kWave - 1);
  float v[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int idx = lane + kWave * i;
    v[i] = logits[idx < E ? idx : E - 1];
  }
  uint64_t key[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int idx = lane + kWave * i;
    const uint32_t b = __float_as_uint(v[i]);
    const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    const bool ok = idx < E && !__builtin_isnan(v[i]);
    key[i] = ok ? (((uint64_t)ord << 32) | (uint32_t)(~idx)) : 0ull;
  }
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j >= k) break;
    uint64_t mine = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) mine = key[i] > mine ? key[i] : mine;
    const uint64_t win = wave_max_u64(mine);
    if (win == 0) {
      ids[j] = -1;
      vals[j] = 0.f;
      continue;
    }
    const int idx = (int)(~(uint32_t)win);
    const uint32_t ord = (uint32_t)(win >> 32);
    ids[j] = idx;
    vals[j] = __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
    if ((idx & (kWave - 1)) == lane) {
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (i == idx / kWave) key[i] = 0;
    }
  }
  const float m = vals[0];
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j >= k) break;
    w[j] = ids[j] >= 0 ? expf(vals[j] - m) : 0.f;
    sum += w[j];
  }
  const float inv = 1.f / sum;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j >= k) break;
    w[j] = w[j] * inv;
  }
}

__device__ __forceinline__ void wave_topk(const float* __restrict__ logits, int E, int k,
                                          int* ids, float* vals, float* w) {
  if (E <= 512)
    wave_topk_n<8>(logits, E, k, ids, vals, w);
  else
    wave_topk_n<16>(logits, E, k, ids, vals, w);
}

// Keeps the compiler from moving instructions across this point (issue order of memory
// operations matters: the in-order vmcnt counter makes a wait on an early load cheap only
// if later weight loads were issued after it).
__device__ __forceinline__ void issue_fence() { __builtin_amdgcn_sched_barrier(0); }

__device__ __forceinline__ float sigmoidf_acc(float a) {
  return __builtin_amdgcn_rcpf(1.f + __expf(-a));
}
__device__ __forceinline__ float siluf_acc(float g) { return g * __builtin_amdgcn_rcpf(1.f + __expf(-g)); }

// Block-wide sum for blockDim.x <= 1024; every thread gets the result. `red` holds >= 16 floats.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = seg_sum<kWave>(v);
  const int wave = threadIdx.x / kWave;
  const int nw = (blockDim.x + kWave - 1) / kWave;
  __syncthreads();
  if ((threadIdx.x & (kWave - 1)) == 0) red[wave] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}

}  // namespace moe
