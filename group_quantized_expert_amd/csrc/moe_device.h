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

// w & mask, opaque to the optimizer: keeps the following byte extracts as single
// v_cvt_f32_ubyte{0..3} instead of a bit-field extract plus a conversion each.
__device__ __forceinline__ uint32_t and_opaque(uint32_t w, uint32_t mask) {
  uint32_t r;
  asm("v_and_b32 %0, %1, %2" : "=v"(r) : "s"(mask), "v"(w));
  return r;
}

// sum(code_i * x_i) over one 16-byte chunk of q4 codes; x in natural element order.
// Element 2j sits in the low nibble of byte j, 2j+1 in the high nibble.
__device__ __forceinline__ float dot_chunk_q4(const uint4 c, const float* __restrict__ x) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  float acc = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t lo = and_opaque(w[d], 0x0F0F0F0Fu);        // elements 8d + 0, 2, 4, 6
    const uint32_t hi = and_opaque(w[d] >> 4, 0x0F0F0F0Fu);   // elements 8d + 1, 3, 5, 7
    const float* xd = x + 8 * d;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc = fmaf((float)((lo >> (8 * j)) & 0xFFu), xd[2 * j], acc);
      acc = fmaf((float)((hi >> (8 * j)) & 0xFFu), xd[2 * j + 1], acc);
    }
  }
  return acc;
}

// sum(code_i * x_i) over one 16-byte chunk of q2 codes; element c at bits 2*(c%4) of byte c/4.
__device__ __forceinline__ float dot_chunk_q2(const uint4 c, const float* __restrict__ x) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  float acc = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const float* xd = x + 16 * d;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t f = and_opaque(w[d] >> (2 * m), 0x03030303u);  // elements 16d + 4j + m
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = fmaf((float)((f >> (8 * j)) & 0xFFu), xd[4 * j + m], acc);
    }
  }
  return acc;
}

template <int BITS>
__device__ __forceinline__ float dot_chunk(const uint4 c, const float* __restrict__ x) {
  if constexpr (BITS == 4)
    return dot_chunk_q4(c, x);
  else
    return dot_chunk_q2(c, x);
}

// Sum over aligned segments of W lanes (W a power of two <= 64); every lane gets its segment sum.
template <int W>
__device__ __forceinline__ float seg_sum(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Per-lane view of one quantized matrix row set: which chunk positions the lane owns.
template <int BITS, int C>
struct LaneRow {
  using G = Geo<BITS, C>;
  int sub;                       // row within the wave's pass
  int chunk[G::kPasses];         // chunk index within the row, per pass
  float x[G::kXPerLane];         // inputs of the owned chunks
  float xsum[G::kPasses];        // per-chunk input sums

  __device__ __forceinline__ void init(int lane, const float* __restrict__ xin, float scale) {
    sub = lane / G::kLanesPerRow;
#pragma unroll
    for (int p = 0; p < G::kPasses; ++p) {
      chunk[p] = (lane % G::kLanesPerRow) + G::kLanesPerRow * p;
      const float4* src = reinterpret_cast<const float4*>(xin + chunk[p] * G::kCodesPerChunk);
      float s = 0.f;
#pragma unroll
      for (int v = 0; v < G::kCodesPerChunk / 4; ++v) {
        float4 t = src[v];
        float* d = x + p * G::kCodesPerChunk + 4 * v;
        d[0] = t.x * scale;
        d[1] = t.y * scale;
        d[2] = t.z * scale;
        d[3] = t.w * scale;
        s += d[0] + d[1] + d[2] + d[3];
      }
      xsum[p] = s;
    }
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
      q[p] = *reinterpret_cast<const uint4*>(codes + lr.chunk[p] * 16);
      const int gi = row * G::kGroupsPerRow + lr.chunk[p] / G::kChunksPerGroup;
      s[p] = scale[gi];
      b[p] = bias[gi];
    }
  }

  // this lane's partial of the row dot product
  __device__ __forceinline__ float partial(const LaneRow<BITS, C>& lr) const {
    float acc = 0.f;
#pragma unroll
    for (int p = 0; p < G::kPasses; ++p) {
      const float qx = dot_chunk<BITS>(q[p], lr.x + p * G::kCodesPerChunk);
      acc += bf16f(s[p]) * qx + bf16f(b[p]) * lr.xsum[p];
    }
    return acc;
  }
};

// One-wave top-k over E <= 1024 logits (ties to the lower index, NaN never chosen),
// renormalised softmax weights over the selected.  All lanes return the same values in
// ids/vals/w, which must hold kMaxTopK entries; entries >= k are left untouched.
// ids[j] = -1 and w[j] = 0 when fewer than j+1 logits are selectable.
constexpr int kMaxTopK = 8;

__device__ __forceinline__ void wave_topk(const float* __restrict__ logits, int E, int k,
                                          int* ids, float* vals, float* w) {
  const int lane = threadIdx.x & (kWave - 1);
  constexpr int kMaxPer = 16;
  constexpr int kNone = 0x7FFFFFFF;
  float v[kMaxPer];
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int idx = lane + kWave * i;
    v[i] = idx < E ? logits[idx] : __builtin_nanf("");
  }
  uint32_t taken = 0;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j >= k) break;
    float bv = 0.f;
    int bi = kNone;
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      const bool ok = !((taken >> i) & 1u) && !__builtin_isnan(v[i]);
      if (ok && (bi == kNone || v[i] > bv)) {
        bv = v[i];
        bi = lane + kWave * i;
      }
    }
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      const bool better = oi != kNone && (bi == kNone || ov > bv || (ov == bv && oi < bi));
      if (better) {
        bv = ov;
        bi = oi;
      }
    }
    ids[j] = bi == kNone ? -1 : bi;
    vals[j] = bv;
    if (bi != kNone && (bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
  }
  const float m = vals[0];
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j >= k) break;
    w[j] = ids[j] >= 0 ? expf(vals[j] - m) : 0.f;
    sum += w[j];
  }
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j >= k) break;
    w[j] = w[j] / sum;
  }
}

__device__ __forceinline__ float sigmoidf_acc(float a) { return 1.f / (1.f + expf(-a)); }
__device__ __forceinline__ float siluf_acc(float g) { return g / (1.f + expf(-g)); }

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
