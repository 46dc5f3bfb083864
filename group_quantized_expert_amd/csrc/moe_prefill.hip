// moe_prefill.hip -- batched (prefill) path of libmoe: T tokens through one MoE layer.
//
// Same arithmetic as the decode layer for every token (router logits, top-k with
// renormalised softmax weights, sigmoid shared gate, per-expert SwiGLU FFN, weighted
// combine + residual), reorganised for many tokens:
//   P0  per token: x -> fp16 hi/lo split (MFMA operands), per-group sums of x, and the
//       shared-gate logit w_sg . x
//   P1  router logits X W_r^T on fp32 MFMA
//   P2  top-k per token (one wave per token)
//   P3  counting sort of the (token, slot) pairs by expert, one block: histogram,
//       exclusive scan, scatter; cut every expert's rows (and the shared expert's token
//       rows) into segments of at most 32 rows
//   P4  grouped gate/up dequant GEMM + SwiGLU per segment on MFMA (fp16 inputs, fp32
//       accumulation); the per-group scale and bias are applied to each group's partial
//       sum: s * sum(q * x) + b * sum(x)
//   P4b intermediate activations -> fp16 hi/lo + per-group sums
//   P5  grouped down dequant GEMM per segment on MFMA
//   P6  per-token gather-combine through the inverse permutation (no atomics, so the
//       result does not depend on the order the sort placed rows in)
// The pages describe only single-token decode; this batched organisation is the
// grouped-GEMM form of the same per-token computation.
//
// Precision: activations are split as x = hi + lo with hi = fp16(x), lo = fp16(x - hi)
// (about 22 significant bits), codes 0..15 are exact in fp16, and every MFMA product of
// a code and an fp16 value is exact in the fp32 accumulator.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"
#include "moe_device.h"
#include "moe_host.h"

namespace moe {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kSegRows = 32;     // rows per segment (one 32-row MFMA tile)
constexpr int kGuChunk = 256;    // h columns per gate/up block (8 waves x 32)
constexpr int kDnChunk = 512;    // output columns per down block (8 waves x 64)

struct Seg {
  int slot, row0, nrows, pad;
};

// Element order of an fp16 MFMA operand vector built from one dword of q4 codes: the
// converter yields [q0 q2 q4 q6 q1 q3 q5 q7]; activations are stored in the same order
// inside every aligned block of 8 so the k indices of the two operands match.
__device__ __forceinline__ constexpr int perm8(int i) { return i < 4 ? 2 * i : 2 * (i - 4) + 1; }

// 8 q4 codes (element i in nibble i) -> fp16 operand [q0 q2 q4 q6 q1 q3 q5 q7].
// A code byte b read as FP8 E4M3 is b * 2^-9; the converter's scale 512 makes it b.
__device__ __forceinline__ h8 codes8_f16(uint32_t w) {
  const uint32_t lo = w & 0x0F0F0F0Fu;
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;
  const h2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)lo, 512.f, false);  // q0 q2
  const h2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)lo, 512.f, true);   // q4 q6
  const h2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)hi, 512.f, false);  // q1 q3
  const h2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)hi, 512.f, true);   // q5 q7
  h8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

__device__ __forceinline__ h8 ld_h8(const _Float16* p) {
  return *reinterpret_cast<const h8*>(p);
}

// ------------------------------------------------------------------------------------------
// P0: split x into fp16 hi/lo (permuted blocks of 8), per-group sums, shared-gate logit.
// One block (256 threads) per token.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prep_x_kernel(const float* __restrict__ x, int H,
                                                     const float* __restrict__ w_sg,
                                                     _Float16* __restrict__ xh,
                                                     _Float16* __restrict__ xl,
                                                     float* __restrict__ xs,
                                                     float* __restrict__ sg_logit) {
  __shared__ float red[16];
  const int t = blockIdx.x;
  const float* xr = x + (size_t)t * H;
  float dot = 0.f;
  // each thread handles blocks of 8 consecutive elements; 8 threads cover a group of 64
  for (int b8 = threadIdx.x; b8 < H / 8; b8 += blockDim.x) {
    const float4 v0 = reinterpret_cast<const float4*>(xr)[2 * b8];
    const float4 v1 = reinterpret_cast<const float4*>(xr)[2 * b8 + 1];
    const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    h8 hv, lv;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float e = v[perm8(i)];
      const _Float16 h = (_Float16)e;
      hv[i] = h;
      lv[i] = (_Float16)(e - (float)h);
      s += v[i];
    }
    *reinterpret_cast<h8*>(xh + (size_t)t * H + 8 * b8) = hv;
    *reinterpret_cast<h8*>(xl + (size_t)t * H + 8 * b8) = lv;
    // group sum over the 8 threads sharing the group (lanes 8j..8j+7 of a wave)
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    s += __shfl_xor(s, 4, 64);
    if ((b8 & 7) == 0) xs[(size_t)t * (H / 64) + b8 / 8] = s;
    if (w_sg) {
      const float4 w0 = reinterpret_cast<const float4*>(w_sg)[2 * b8];
      const float4 w1 = reinterpret_cast<const float4*>(w_sg)[2 * b8 + 1];
      dot = fmaf(w0.x, v0.x, dot); dot = fmaf(w0.y, v0.y, dot);
      dot = fmaf(w0.z, v0.z, dot); dot = fmaf(w0.w, v0.w, dot);
      dot = fmaf(w1.x, v1.x, dot); dot = fmaf(w1.y, v1.y, dot);
      dot = fmaf(w1.z, v1.z, dot); dot = fmaf(w1.w, v1.w, dot);
    }
  }
  if (w_sg) {
    dot = block_sum(dot, red);
    if (threadIdx.x == 0) sg_logit[t] = dot;
  }
}

// ------------------------------------------------------------------------------------------
// P1: logits[t][e] = x[t] . w_router[e] with fp32 MFMA 16x16x4.  Block: 64 tokens x 64
// router rows.  Lane (m = l%16, c = l/16) feeds k = k0 + 4c + j to MFMA j of each 16-wide k
// step.
// ------------------------------------------------------------------------------------------
// Measured: when every wave loaded the block's 64 router rows itself (four times the L1
// traffic) the kernel took 0.20 ms; staging the router rows through LDS, 0.14 ms; staging the
// token rows too, with 8 waves instead of 4, 0.12 ms.  An fp16 hi/lo split of both operands on
// f16 MFMA was only 11 % faster than fp32 (the kernel is bound by its loads), so the router
// stays exact fp32.  Rows are padded to 68 floats so that the 16 rows read by a fragment fall
// into distinct banks.
constexpr int kRgK = 64;        // k per chunk
constexpr int kRgRow = kRgK + 4;
// 8 waves: wave w takes tokens 16 (w % 4) .. + 15 against router rows 32 (w / 4) .. + 31 (two
// 16x16 tiles); both the block's 64 token rows and its 64 router rows are staged through LDS
// (8 floats of each per thread and chunk), so each is read from L2 once per block.
// Block z of gridDim.z takes k in [z kz_len, (z + 1) kz_len) and, when the k range is split
// (gridDim.z > 1), writes its partial sums to part[z][t][e] for router_reduce_kernel.
__global__ __launch_bounds__(512) void router_gemm_kernel(const float* __restrict__ x, int T,
                                                          int H, const float* __restrict__ w,
                                                          int E, int kz_len,
                                                          float* __restrict__ logits,
                                                          float* __restrict__ part) {
  constexpr int NT = 2;
  __shared__ __attribute__((aligned(16))) float xs[2][64][kRgRow];
  __shared__ __attribute__((aligned(16))) float ws[2][64][kRgRow];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, c = lane >> 4;
  const int tg = wave & 3, eh = wave >> 2;
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  // staging map: thread -> row tid / 8 of both tiles, floats 8 (tid % 8) .. + 7 of the chunk
  const int sr = tid >> 3, sp = 8 * (tid & 7);
  const int kz0 = blockIdx.z * kz_len;
  const float* xr = x + (size_t)(t0 + sr < T ? t0 + sr : T - 1) * H + kz0 + sp;
  const float* wr = w + (size_t)(e0 + sr) * H + kz0 + sp;
  const int nch = kz_len / kRgK;
  f4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f4{0.f, 0.f, 0.f, 0.f};
  float4 xv0, xv1, wv0, wv1;
  auto load = [&](int ch) {
    xv0 = *reinterpret_cast<const float4*>(xr + ch * kRgK);
    xv1 = *reinterpret_cast<const float4*>(xr + ch * kRgK + 4);
    wv0 = ld_nt_f4(wr + ch * kRgK);
    wv1 = ld_nt_f4(wr + ch * kRgK + 4);
  };
  auto store = [&](int buf) {
    *reinterpret_cast<float4*>(&xs[buf][sr][sp]) = xv0;
    *reinterpret_cast<float4*>(&xs[buf][sr][sp + 4]) = xv1;
    *reinterpret_cast<float4*>(&ws[buf][sr][sp]) = wv0;
    *reinterpret_cast<float4*>(&ws[buf][sr][sp + 4]) = wv1;
  };
  auto compute = [&](int buf) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float4 a = *reinterpret_cast<const float4*>(&xs[buf][16 * tg + m][16 * s + 4 * c]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float4 b = *reinterpret_cast<const float4*>(&ws[buf][32 * eh + 16 * nt + m][16 * s + 4 * c]);
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, acc[nt], 0, 0, 0);
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, acc[nt], 0, 0, 0);
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, acc[nt], 0, 0, 0);
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, acc[nt], 0, 0, 0);
      }
    }
  };
  // one chunk ahead; the last chunk reloads itself so that every step issues the same loads
  load(0);
  store(0);
  __syncthreads();
#pragma unroll 1
  for (int ch = 0; ch < nch; ++ch) {
    load(ch + 1 < nch ? ch + 1 : ch);
    __builtin_amdgcn_sched_barrier(0);
    compute(ch & 1);
    store((ch + 1) & 1);
    __syncthreads();
  }
  // D layout: lane holds rows 4c+i (tokens) of column m (router row)
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tt = t0 + 16 * tg + 4 * c + i;
      float* dst = gridDim.z > 1 ? part + (size_t)blockIdx.z * T * E : logits;
      if (tt < T) dst[(size_t)tt * E + e0 + 32 * eh + 16 * nt + m] = acc[nt][i];
    }
}

// Sum of the k-range partials in a fixed order (the result does not depend on the launch).
// All KS partials are loaded before the first add (one memory latency, not KS of them).
template <int KS>
__global__ __launch_bounds__(256) void router_reduce_kernel(const float* __restrict__ part, int n,
                                                            float* __restrict__ logits) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float v[KS];
#pragma unroll
  for (int z = 0; z < KS; ++z) v[z] = part[(size_t)z * n + i];
  float s = v[0];
#pragma unroll
  for (int z = 1; z < KS; ++z) s += v[z];
  logits[i] = s;
}

// Few tokens leave few 64 x 64 router blocks (8 at T <= 64 with E = 512), each streaming its
// 64 rows over the whole k: split the k range until there are as many blocks as compute units
// (256), keeping >= 2 chunks of 64 k per block.  (At 2048 tokens there are 256 blocks already.)
inline int router_ksplit(int T, int E, int H) {
  const int blocks = ((T + 63) / 64) * (E / 64);
  int ks = 1;
  while (blocks * ks < 256 && ks < 32 && H / (2 * ks) >= 2 * kRgK) ks *= 2;
  return ks;
}

// ------------------------------------------------------------------------------------------
// P2: top-k per token (one wave), sg = sigmoid(sg_logit).
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(64) void prefill_topk_kernel(const float* __restrict__ logits,
                                                          int E, int k,
                                                          const float* __restrict__ sg_logit,
                                                          int32_t* ids, float* wts, float* sg,
                                                          int32_t* ids_out, float* wts_out,
                                                          float* sg_out) {
  const int t = blockIdx.x;
  int id[kMaxTopK];
  float vals[kMaxTopK], w[kMaxTopK];
  wave_topk(logits + (size_t)t * E, E, k, id, vals, w);
  if (threadIdx.x == 0) {
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j >= k) break;
      ids[(size_t)t * k + j] = id[j];
      wts[(size_t)t * k + j] = w[j];
      if (ids_out) ids_out[(size_t)t * k + j] = id[j];
      if (wts_out) wts_out[(size_t)t * k + j] = w[j];
    }
    const float g = sg_logit ? sigmoidf_acc(sg_logit[t]) : 1.f;
    sg[t] = g;
    if (sg_out) sg_out[t] = g;
  }
}

// ------------------------------------------------------------------------------------------
// P3: sort (token, slot) pairs by expert (one block of 1024 threads).  Row space: routed
// pairs occupy rows [0, T*k) in expert order, the shared expert's tokens rows
// [T*k, T*k + T).  a_row[r] = token whose activations row r reads; inv[t*k+j] = row of
// pair (t, j) (-1 when the pair has no expert).  Segments of <= kSegRows rows.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void sort_kernel(const int32_t* __restrict__ ids, int T,
                                                    int k, int E, int shared_slot,
                                                    int32_t* __restrict__ a_row,
                                                    int32_t* __restrict__ inv,
                                                    Seg* __restrict__ segs,
                                                    int32_t* __restrict__ nseg) {
  __shared__ int cnt[1024];
  __shared__ int off[1024];
  __shared__ int wsum[16];
  __shared__ int total_segs;
  const int tid = threadIdx.x;
  const int np = T * k;
  for (int e = tid; e < 1024; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  for (int p = tid; p < np; p += blockDim.x) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  // exclusive scans over experts (one expert per thread): row offsets and segment offsets
  const int n_e = tid < E ? cnt[tid] : 0;
  const int sg_e = (n_e + kSegRows - 1) / kSegRows;
  auto block_exclusive_scan = [&](int v) {
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o, 64);
      if ((tid & 63) >= o) incl += u;
    }
    __syncthreads();
    if ((tid & 63) == 63) wsum[tid >> 6] = incl;
    __syncthreads();
    int base = 0;
    for (int i = 0; i < (tid >> 6); ++i) base += wsum[i];
    return base + incl - v;
  };
  const int row_off = block_exclusive_scan(n_e);
  const int seg_off = block_exclusive_scan(sg_e);
  if (tid < E) off[tid] = row_off;
  if (tid == E - 1) total_segs = seg_off + sg_e;
  if (tid < E)
    for (int s = 0; s < sg_e; ++s) {
      const int r0 = row_off + s * kSegRows;
      const int n = (n_e - s * kSegRows) < kSegRows ? (n_e - s * kSegRows) : kSegRows;
      segs[seg_off + s] = Seg{tid, r0, n, 0};
    }
  __syncthreads();
  // scatter pairs into expert order (order inside an expert is not significant)
  for (int p = tid; p < np; p += blockDim.x) {
    const int e = ids[p];
    if (e >= 0 && e < E) {
      const int pos = atomicAdd(&off[e], 1);
      a_row[pos] = p / k;
      inv[p] = pos;
    } else {
      inv[p] = -1;
    }
  }
  // shared expert rows: token t at row T*k + t
  const int base = total_segs;
  const int nsh = shared_slot >= 0 ? (T + kSegRows - 1) / kSegRows : 0;
  for (int t = tid; t < (shared_slot >= 0 ? T : 0); t += blockDim.x) a_row[np + t] = t;
  for (int s = tid; s < nsh; s += blockDim.x) {
    const int n = (T - s * kSegRows) < kSegRows ? (T - s * kSegRows) : kSegRows;
    segs[base + s] = Seg{shared_slot, np + s * kSegRows, n, 0};
  }
  if (tid == 0) *nseg = base + nsh;
}

// ------------------------------------------------------------------------------------------
// Grouped dequant GEMM core on MFMA 32x32x16 f16.  A block (8 waves) computes the (up to 32)
// rows of one segment against 8 x NT column tiles of 32; wave w owns NT column tiles.  Over
// K = C (groups of 64):
//   out[r][n] = sum_g ( s[n][g] * sum_{k in g} q[n][k] a[r][k] + b[n][g] * asum[r][g] )
// The first term runs in chunks of CG groups: the block stages the chunk's activation rows
// (fp16 hi and lo) in double-buffered LDS, while every wave holds the next chunk's codes in
// registers, so HBM streams the weights continuously.  The bias term is a separate small
// product over the groups (see grouped_tile).  Measured choices:
//  - a chunk reads 32 CG bytes of each weight row: with CG = 4 one whole 128-byte line, so no
//    line has to stay in L2 from one chunk to the next (gate/up rows 2 KB apart map to few
//    L2 sets: 2-group chunks read 13.6 instead of 2.8 GB);
//  - a chunk's code loads are issued together: refilling each group's registers as soon as it
//    was multiplied split the lines into separate L1 misses (2.6 times the L2 requests, and
//    the down kernel's half-line chunks read 1.9 instead of 1.3 GB);
//  - the 32x32 tile lets each lane read 16 code bytes per group (two lanes per row); the 16x16
//    tile's 8-byte reads (four lanes per row) streamed measurably slower;
//  - more column tiles per wave mean fewer blocks reading the same activation rows: two tiles
//    per gate/up wave instead of one took 7 % less time;
//  - the scales are staged in LDS once for the whole K with 16-byte loads: fetched per chunk
//    as 4-byte gathers they cost a fifth of the kernel time.
// ------------------------------------------------------------------------------------------
// The 16-byte slots of a row are stored XOR-swizzled by the row (slot s of row r at s ^ (r mod
// 16)): the lanes of a fragment read the same slot of consecutive rows, which a plain
// power-of-two row length would put in one bank group (measured: 16-byte row padding still
// leaves half the cycles in bank conflicts, the swizzle none).  The struct is 16-byte aligned,
// or the compiler splits each 16-byte fragment read into 4-byte reads.
template <int CG>
struct __attribute__((aligned(16))) ASmem {
  _Float16 a[2][2][kSegRows][64 * CG];  // [buffer][hi, lo][row][k, slots swizzled]
};
__device__ __forceinline__ int aslot(int row, int slot) { return 8 * (slot ^ (row & 15)); }

template <int NT, int CG>
struct BChunk {
  uint4 q[NT][CG];  // 16 code bytes per lane per 32-row tile and group
};

// Scales of every wave's tiles over the whole K, staged once per block: per wave and 16-row
// region 16 rows of G bf16, rows padded by 8 bytes so that the rows read by a fragment fall
// into distinct banks.
template <int NT, int G>
struct MSmem {
  static constexpr int kRow = 2 * G + 8;
  uint8_t m[8][NT][16][kRow];
};

typedef float f16v __attribute__((ext_vector_type(16)));

// tile_rec[rg], tile_row[rg]: matrix record and first weight row (uniform) of 16-row region
// rg; region 2t + h holds rows 16h .. 16h + 15 of the wave's 32-row tile t.
// MFMA 32x32x16 f16: lane l = (n = l % 32, u = l / 32) feeds activation row n and weight row n
// of the tile; k step j of group g takes the group's k = 32 u + 8 j .. + 7 from both, which
// for the weights is dword j of one 16-byte load (bytes 16 u .. 16 u + 15 of the group).
// Result: lane (n, u) holds out[8 b + 4 u + t][n] in element 4 b + t.
template <int NR, int C, int CG>
__device__ __forceinline__ void grouped_tile(const uint8_t* const* tile_rec, const int* tile_row,
                                             int R_w, const _Float16* __restrict__ ah,
                                             const _Float16* __restrict__ al,
                                             const float* __restrict__ asum,
                                             const int* __restrict__ row_index,  // or null
                                             int row0, int nrows, ASmem<CG>& sm,
                                             MSmem<NR, C / 64>& msm, f16v (&tot)[NR / 2]) {
  constexpr int NT = NR / 2;  // 32-row tiles per wave
  constexpr int G = C / 64;
  constexpr int NCH = G / CG;
  constexpr int kChunkK = 64 * CG;
  constexpr int kStage = CG / 2;  // 16-byte activation parts per thread and operand half
  constexpr size_t kRowBytes = C / 2;
  static_assert(G % CG == 0 && CG % 2 == 0 && CG <= 16 && NR % 2 == 0, "");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int n = lane & 31, u = lane >> 5;
  const int hf = n >> 4, nr = n & 15;

  // uniform region bases; per lane: the code and scale/bias rows of weight row n of each tile
  const uint16_t* sbase[NR];
#pragma unroll
  for (int rg = 0; rg < NR; ++rg)
    sbase[rg] = reinterpret_cast<const uint16_t*>(tile_rec[rg] + (size_t)R_w * kRowBytes) +
                (size_t)tile_row[rg] * G;
  const uint8_t* crow[NT];
  const uint16_t* brow[NT];
  const size_t bias_delta = (size_t)R_w * G;  // bias plane follows the scale plane
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const uint8_t* c0 = tile_rec[2 * t] + (size_t)(tile_row[2 * t] + nr) * kRowBytes;
    const uint8_t* c1 = tile_rec[2 * t + 1] + (size_t)(tile_row[2 * t + 1] + nr) * kRowBytes;
    crow[t] = (hf ? c1 : c0) + 16 * u;
    brow[t] = (hf ? sbase[2 * t + 1] : sbase[2 * t]) + bias_delta + nr * G;
  }

  // activation staging map: thread -> (row, 16-byte parts spart + 16 i); 512 threads cover 32
  // rows x 64 CG halves for hi and lo.  Rows past the segment are staged with row 0's values:
  // their MFMA output rows are discarded, and no other row depends on them.
  const int srow = tid >> 4, spart = tid & 15;
  const bool srow_ok = srow < nrows;
  const int sr = srow_ok ? srow : 0;
  const size_t arow = (size_t)(row_index ? row_index[row0 + sr] : row0 + sr);
  const _Float16* ahr = ah + arow * C + 8 * spart;
  const _Float16* alr = al + arow * C + 8 * spart;

  // issued and stored by every thread (rows past the segment hold row 0's values, whose
  // outputs are discarded): with no branch around them the compiler keeps the loads where
  // they are issued, ahead of the chunk's arithmetic, and its waits count them exactly
  auto load_a = [&](int ch, h8 (&vh)[kStage], h8 (&vl)[kStage]) {
    const int k0 = ch * kChunkK;
#pragma unroll
    for (int i = 0; i < kStage; ++i) {
      vh[i] = ld_h8(ahr + k0 + 128 * i);
      vl[i] = ld_h8(alr + k0 + 128 * i);
    }
  };
  auto store_a = [&](int buf, const h8 (&vh)[kStage], const h8 (&vl)[kStage]) {
#pragma unroll
    for (int i = 0; i < kStage; ++i) {
      *reinterpret_cast<h8*>(&sm.a[buf][0][srow][aslot(srow, 16 * i + spart)]) = vh[i];
      *reinterpret_cast<h8*>(&sm.a[buf][1][srow][aslot(srow, 16 * i + spart)]) = vl[i];
    }
  };
  // one 16-byte load per lane, tile and group: 32 rows x 32 bytes
  auto load_b = [&](int ch, BChunk<NT, CG>& bc) {
    const int g0 = ch * CG;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int gi = 0; gi < CG; ++gi)
        bc.q[t][gi] = *reinterpret_cast<const uint4*>(crow[t] + 32 * (g0 + gi));
  };
  // scale staging: the wave's NR regions of 16 rows x G bf16 are contiguous in memory per
  // region (consecutive rows); units of kU bytes (16, or 8 when a row is shorter)
  constexpr int kMRow = MSmem<NR, G>::kRow;
  constexpr int kU = (G % 8 == 0) ? 16 : 8;
  constexpr int kUR = 2 * G / kU;       // units per row
  constexpr int kUnits = 16 * kUR;      // units per region
  constexpr int kMLoads = (kUnits + 63) / 64;  // per region (lanes past kUnits idle)
  static_assert(G % 4 == 0, "");
  const int wave = tid >> 6;
  uint8_t* mw = &msm.m[wave][0][0][0];
  uint4 mv[NR][kMLoads];
  auto load_meta = [&]() {
#pragma unroll
    for (int rg = 0; rg < NR; ++rg)
#pragma unroll
      for (int i = 0; i < kMLoads; ++i) {
        const int v = 64 * i + lane, row = v / kUR, part = v % kUR;
        if (v < kUnits) {
          if constexpr (kU == 16) {
            mv[rg][i] = *reinterpret_cast<const uint4*>(sbase[rg] + row * G + 8 * part);
          } else {
            const uint2 w = *reinterpret_cast<const uint2*>(sbase[rg] + row * G + 4 * part);
            mv[rg][i] = make_uint4(w.x, w.y, 0u, 0u);
          }
        }
      }
  };
  auto store_meta = [&]() {
#pragma unroll
    for (int rg = 0; rg < NR; ++rg)
#pragma unroll
      for (int i = 0; i < kMLoads; ++i) {
        const int v = 64 * i + lane, row = v / kUR, part = v % kUR;
        if (v < kUnits) {
          uint2* d = reinterpret_cast<uint2*>(mw + (rg * 16 + row) * kMRow + kU * part);
          d[0] = make_uint2(mv[rg][i].x, mv[rg][i].y);
          if constexpr (kU == 16) d[1] = make_uint2(mv[rg][i].z, mv[rg][i].w);
        }
      }
  };
  auto compute = [&](int buf, int ch, const BChunk<NT, CG>& bc) {
    uint32_t msw[NT][CG / 2];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint8_t* ms = mw + ((2 * t + hf) * 16 + nr) * kMRow + 2 * CG * ch;
      if constexpr (CG == 4) {
        const uint2 a = *reinterpret_cast<const uint2*>(ms);
        msw[t][0] = a.x; msw[t][1] = a.y;
      } else {
#pragma unroll
        for (int w = 0; w < CG / 2; ++w) msw[t][w] = *reinterpret_cast<const uint32_t*>(ms + 4 * w);
      }
    }
#pragma unroll
    for (int gi = 0; gi < CG; ++gi) {
      h8 a_h[4], a_l[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a_h[j] = *reinterpret_cast<const h8*>(&sm.a[buf][0][n][aslot(n, 8 * gi + 4 * u + j)]);
        a_l[j] = *reinterpret_cast<const h8*>(&sm.a[buf][1][n][aslot(n, 8 * gi + 4 * u + j)]);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint32_t sw = msw[t][gi >> 1];
        const float sc = __uint_as_float((gi & 1) ? (sw & 0xFFFF0000u) : (sw << 16));
        const uint4 q = bc.q[t][gi];
        const h8 b0 = codes8_f16(q.x), b1 = codes8_f16(q.y), b2 = codes8_f16(q.z), b3 = codes8_f16(q.w);
        f16v acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_h[0], b0, f16v{}, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_h[1], b1, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_h[2], b2, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_h[3], b3, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_l[0], b0, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_l[1], b1, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_l[2], b2, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_l[3], b3, acc, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 16; ++e) tot[t][e] = fmaf(sc, acc[e], tot[t][e]);
      }
    }
  };

  // activation rows and weights are loaded one chunk ahead (two register buffers for the
  // weights, so the steps come in pairs with static names); the LDS buffer alternates by chunk
  h8 avh[kStage], avl[kStage];
  auto step = [&](int ch, const BChunk<NT, CG>& cur, BChunk<NT, CG>& next) {
    // the last step reloads its own chunk (cache hits) instead of branching around the loads:
    // with the same loads on every path the compiler's waits count them exactly
    const int nx = ch + 1 < NCH ? ch + 1 : ch;
    // The loads, and below the LDS stores, run at a raised issue priority: with the default
    // arbitration by age the older wave of a SIMD starts its products while the younger one
    // has not issued its loads yet, and those loads then go out a chunk's arithmetic late.
    __builtin_amdgcn_s_setprio(1);
    load_a(nx, avh, avl);
    load_b(nx, next);
    __builtin_amdgcn_s_setprio(0);
    // keep the next chunk's loads ahead of this chunk's arithmetic
    __builtin_amdgcn_sched_barrier(0);
    compute(ch & 1, ch, cur);
    // unconditional too (the last step rewrites a buffer nobody reads again): a conditional
    // store would let the compiler sink the activation loads into its branch, after compute
    __builtin_amdgcn_s_setprio(1);
    store_a((ch + 1) & 1, avh, avl);
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();
  };
  // The bias part, sum_g b[n][g] asum[r][g], is one more product over K = G on bf16 MFMA
  // 32x32x16: the bf16 biases enter exactly and the fp32 group sums as three bf16 parts (24
  // bits), so every product is exact and only the fp32 accumulation rounds.  Lane (n, u)
  // feeds groups 16 j + 8 u .. + 7 of activation row n and of weight row n.  Its result is
  // the starting value of tot.
  typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
  constexpr int KS = (G + 15) / 16;
  uint4 bias_v[KS][NT];
  float4 asum_v[KS][2];
  const bool n_ok = n < nrows;
  const float* arow_sum = asum + (size_t)(row_index ? row_index[row0 + (n_ok ? n : 0)] : row0 + n) * G;
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    const int g0 = 16 * j + 8 * u;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint16_t* bp = brow[t] + g0;
      if constexpr (G % 8 == 0) {
        bias_v[j][t] = g0 < G ? *reinterpret_cast<const uint4*>(bp) : make_uint4(0u, 0u, 0u, 0u);
      } else {
        uint32_t w[4];
#pragma unroll
        for (int x = 0; x < 4; ++x)
          w[x] = (g0 + 2 * x < G ? (uint32_t)bp[2 * x] : 0u) |
                 (g0 + 2 * x + 1 < G ? (uint32_t)bp[2 * x + 1] << 16 : 0u);
        bias_v[j][t] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = 0.f;
    if (n_ok) {
      const float* ap = arow_sum + g0;
      if constexpr (G % 8 == 0) {
        if (g0 < G) {
          const float4 p = *reinterpret_cast<const float4*>(ap);
          const float4 q = *reinterpret_cast<const float4*>(ap + 4);
          x[0] = p.x; x[1] = p.y; x[2] = p.z; x[3] = p.w;
          x[4] = q.x; x[5] = q.y; x[6] = q.z; x[7] = q.w;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = g0 + e < G ? ap[e] : 0.f;
      }
    }
    asum_v[j][0] = make_float4(x[0], x[1], x[2], x[3]);
    asum_v[j][1] = make_float4(x[4], x[5], x[6], x[7]);
  }
  BChunk<NT, CG> b0c, b1c;
  load_meta();
  load_a(0, avh, avl);
  load_b(0, b0c);
#pragma unroll
  for (int t = 0; t < NT; ++t) tot[t] = f16v{};
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    const float x[8] = {asum_v[j][0].x, asum_v[j][0].y, asum_v[j][0].z, asum_v[j][0].w,
                        asum_v[j][1].x, asum_v[j][1].y, asum_v[j][1].z, asum_v[j][1].w};
    bf8 p0, p1, p2;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const __bf16 h = (__bf16)x[e];
      const float r1 = x[e] - (float)h;
      const __bf16 md = (__bf16)r1;
      p0[e] = h;
      p1[e] = md;
      p2[e] = (__bf16)(r1 - (float)md);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const bf8 b = __builtin_bit_cast(bf8, bias_v[j][t]);
      tot[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(p0, b, tot[t], 0, 0, 0);
      tot[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(p1, b, tot[t], 0, 0, 0);
      tot[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(p2, b, tot[t], 0, 0, 0);
    }
  }
  store_meta();
  store_a(0, avh, avl);
  __syncthreads();
#pragma unroll 1
  for (int ch = 0; ch < NCH; ch += 2) {
    step(ch, b0c, b1c);
    if (ch + 1 >= NCH) break;
    step(ch + 1, b1c, b0c);
  }
}

// ------------------------------------------------------------------------------------------
// P4: gate/up + SwiGLU per segment.  Block (segment, chunk of 256 h columns); wave w owns h
// columns [chunk*256 + 32w, +32): two 32-row tiles, each of 16 gate and the 16 up rows of
// the same h columns.  Blocks
// are ordered so that the column chunks of one segment run back to back on one XCD (block b
// goes to XCD b mod 8), where the segment's activation rows then come from L2.
// ------------------------------------------------------------------------------------------
// NTW tiles per wave: 2 (256 h columns per block) in general; 1 (128 columns, twice the blocks)
// when few tokens leave few segments.
template <int H, int NTW>
__global__ __launch_bounds__(512) void gu_grouped_kernel(const Seg* __restrict__ segs,
                                                         const int32_t* __restrict__ nseg,
                                                         const uint8_t* __restrict__ base,
                                                         int64_t slot_bytes, int I,
                                                         const int32_t* __restrict__ a_row,
                                                         const _Float16* __restrict__ xh,
                                                         const _Float16* __restrict__ xl,
                                                         const float* __restrict__ xs,
                                                         float* __restrict__ hout) {
  constexpr int kChunk = 8 * 16 * NTW;  // h columns per block
  const int nchunk = I / kChunk;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int s = (slot / nchunk) * 8 + xcd, chunk = slot % nchunk;
  if (s >= *nseg) return;
  const Seg sg = segs[s];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h0 = chunk * kChunk + 16 * NTW * wave;
  const uint8_t* rec = base + (size_t)sg.slot * slot_bytes;
  const size_t mat = matrix_rec_bytes<4>(I, H);
  const uint8_t* recs[2 * NTW];
  int wrow[2 * NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    recs[2 * t] = rec;
    recs[2 * t + 1] = rec + mat;
    wrow[2 * t] = wrow[2 * t + 1] = h0 + 16 * t;
  }
  __shared__ ASmem<4> sm;
  __shared__ MSmem<2 * NTW, H / 64> msm;
  f16v tot[NTW];
  grouped_tile<2 * NTW, H, 4>(recs, wrow, I, xh, xl, xs, a_row, sg.row0, sg.nrows, sm, msm, tot);
  // SwiGLU: lane (n, u) holds column n of the 32-row tile for rows 8 b + 4 u + t; columns
  // 0..15 are the gate rows, 16..31 the up rows of the same h columns
  const int n = lane & 31, u = lane >> 5;
#pragma unroll
  for (int t = 0; t < NTW; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float other = __shfl_xor(tot[t][e], 16, 64);
      const int r = 8 * (e >> 2) + 4 * u + (e & 3);
      if (n < 16 && r < sg.nrows)
        hout[(size_t)(sg.row0 + r) * I + h0 + 16 * t + n] = siluf_acc(tot[t][e]) * other;
    }
}

// P4b: h rows -> fp16 hi/lo (permuted blocks of 8) + per-group sums.  One thread per 8
// elements; grid covers all rows.
__global__ __launch_bounds__(256) void prep_h_kernel(const float* __restrict__ h, int R, int I,
                                                     _Float16* __restrict__ hh,
                                                     _Float16* __restrict__ hl,
                                                     float* __restrict__ hs) {
  const size_t b8 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;  // block-of-8 index
  const size_t n8 = (size_t)R * I / 8;
  if (b8 >= n8) return;
  const float4 v0 = reinterpret_cast<const float4*>(h)[2 * b8];
  const float4 v1 = reinterpret_cast<const float4*>(h)[2 * b8 + 1];
  const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  h8 hv, lv;
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float e = v[perm8(i)];
    const _Float16 hi = (_Float16)e;
    hv[i] = hi;
    lv[i] = (_Float16)(e - (float)hi);
    s += v[i];
  }
  *reinterpret_cast<h8*>(hh + 8 * b8) = hv;
  *reinterpret_cast<h8*>(hl + 8 * b8) = lv;
  s += __shfl_xor(s, 1, 64);
  s += __shfl_xor(s, 2, 64);
  s += __shfl_xor(s, 4, 64);
  if ((b8 & 7) == 0) hs[b8 / 8] = s;  // group index = element / 64 = b8 / 8
}

// ------------------------------------------------------------------------------------------
// P5: down per segment.  Block (segment, chunk of 256 output columns); wave w owns output
// columns [chunk*256 + 32w, +32) as one 32-row tile.  (Two tiles per wave, 512 columns per
// block, need 167 VGPRs, so one 8-wave block per CU; one tile at 124 VGPRs lets two blocks
// share a CU and ran ~1 % faster at 2048 tokens.  Four tiles with 2-group chunks, or two with
// 4-group chunks, measured no faster.)
// ------------------------------------------------------------------------------------------
// NTW tiles per wave (the launch uses 1).
template <int I, int NTW>
__global__ __launch_bounds__(512) void dn_grouped_kernel(const Seg* __restrict__ segs,
                                                         const int32_t* __restrict__ nseg,
                                                         const uint8_t* __restrict__ base,
                                                         int64_t slot_bytes, int H,
                                                         const _Float16* __restrict__ hh,
                                                         const _Float16* __restrict__ hl,
                                                         const float* __restrict__ hs,
                                                         float* __restrict__ y) {
  constexpr int kChunk = 8 * 32 * NTW;  // output columns per block
  const int nchunk = H / kChunk;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int s = (slot / nchunk) * 8 + xcd, chunk = slot % nchunk;
  if (s >= *nseg) return;
  const Seg sg = segs[s];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = chunk * kChunk + 32 * NTW * wave;
  const uint8_t* rec = base + (size_t)sg.slot * slot_bytes + 2 * matrix_rec_bytes<4>(I, H);
  const uint8_t* recs[2 * NTW];
  int wrow[2 * NTW];
#pragma unroll
  for (int r = 0; r < 2 * NTW; ++r) {
    recs[r] = rec;
    wrow[r] = n0 + 16 * r;
  }
  __shared__ ASmem<2> sm;
  __shared__ MSmem<2 * NTW, I / 64> msm;
  f16v tot[NTW];
  grouped_tile<2 * NTW, I, 2>(recs, wrow, H, hh, hl, hs, nullptr, sg.row0, sg.nrows, sm, msm, tot);
  const int n = lane & 31, u = lane >> 5;
#pragma unroll
  for (int t = 0; t < NTW; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = 8 * (e >> 2) + 4 * u + (e & 3);
      if (r < sg.nrows) y[(size_t)(sg.row0 + r) * H + n0 + 32 * t + n] = tot[t][e];
    }
}

// ------------------------------------------------------------------------------------------
// P6: out[t] = x[t] + sum_j w[t][j] * y[inv[t*k+j]] + sg[t] * y[T*k + t]; one thread per 4
// columns.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prefill_combine_kernel(
    const float* __restrict__ x, int T, int H, int k, const float* __restrict__ wts,
    const int32_t* __restrict__ inv, const float* __restrict__ sg, int has_shared,
    const float* __restrict__ y, float* __restrict__ out) {
  const int t = blockIdx.y;
  const int c4 = blockIdx.x * blockDim.x + threadIdx.x;
  if (c4 >= H / 4) return;
  float4 o = reinterpret_cast<const float4*>(x + (size_t)t * H)[c4];
  for (int j = 0; j < k; ++j) {
    const int r = inv[(size_t)t * k + j];
    if (r < 0) continue;
    const float w = wts[(size_t)t * k + j];
    const float4 v = reinterpret_cast<const float4*>(y + (size_t)r * H)[c4];
    o.x = fmaf(w, v.x, o.x); o.y = fmaf(w, v.y, o.y);
    o.z = fmaf(w, v.z, o.z); o.w = fmaf(w, v.w, o.w);
  }
  if (has_shared) {
    const float g = sg[t];
    const float4 v = reinterpret_cast<const float4*>(y + ((size_t)T * k + t) * H)[c4];
    o.x = fmaf(g, v.x, o.x); o.y = fmaf(g, v.y, o.y);
    o.z = fmaf(g, v.z, o.z); o.w = fmaf(g, v.w, o.w);
  }
  reinterpret_cast<float4*>(out + (size_t)t * H)[c4] = o;
}

// ------------------------------------------------------------------------------------------
// workspace
// ------------------------------------------------------------------------------------------
struct PrefillWs {
  size_t logits, rpart, sglogit, ids, wts, sg, xh, xl, xs, a_row, inv, segs, nseg, hf, hh, hl, hs, y;
  size_t total;
  int rows, max_segs;
  static PrefillWs make(int T, int H, int I, int E, int k, bool shared) {
    PrefillWs w{};
    w.rows = T * k + (shared ? T : 0);
    w.max_segs = E + (T * k + kSegRows - 1) / kSegRows + (shared ? (T + kSegRows - 1) / kSegRows : 0);
    size_t o = 0;
    auto take = [&](size_t bytes) { const size_t at = o; o = align_up(o + bytes); return at; };
    w.logits = take((size_t)T * E * 4);
    const int ks = router_ksplit(T, E, H);
    w.rpart = take(ks > 1 ? (size_t)ks * T * E * 4 : 0);
    w.sglogit = take((size_t)T * 4);
    w.ids = take((size_t)T * k * 4);
    w.wts = take((size_t)T * k * 4);
    w.sg = take((size_t)T * 4);
    w.xh = take((size_t)T * H * 2);
    w.xl = take((size_t)T * H * 2);
    w.xs = take((size_t)T * (H / 64) * 4);
    w.a_row = take((size_t)w.rows * 4);
    w.inv = take((size_t)T * k * 4);
    w.segs = take((size_t)w.max_segs * sizeof(Seg));
    w.nseg = take(4);
    w.hf = take((size_t)w.rows * I * 4);
    w.hh = take((size_t)w.rows * I * 2);
    w.hl = take((size_t)w.rows * I * 2);
    w.hs = take((size_t)w.rows * (I / 64) * 4);
    w.y = take((size_t)w.rows * H * 4);
    w.total = o;
    return w;
  }
};

bool prefill_shape_ok(const moe_layer* L, int T) {
  const moe_experts& X = L->experts;
  return X.bits == 4 && T >= 1 && T <= 65535 && X.hidden % kDnChunk == 0 &&
         X.inter % kGuChunk == 0 && L->n_experts % 64 == 0 && L->n_experts <= 1024 &&
         (int64_t)T * L->top_k <= (int64_t)1 << 26;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_prefill_workspace_bytes(const moe_layer* layer, int T) {
  if (check_layer(layer) != MOE_OK || !prefill_shape_ok(layer, T)) return 0;
  return PrefillWs::make(T, layer->experts.hidden, layer->experts.inter, layer->n_experts,
                         layer->top_k, layer->shared_slot >= 0).total;
}

moe_status moe_prefill_q4(const moe_layer* layer, const float* x, int T, float* out,
                          int32_t* ids_out, float* weights_out, float* sg_out, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_layer(layer);
  if (st != MOE_OK) return st;
  if (layer->experts.bits != 4) return MOE_E_BITS;
  if (!x || !out) return MOE_E_NULL;
  if (!prefill_shape_ok(layer, T)) return MOE_E_SHAPE;
  if (!aligned16(x) || !aligned16(out)) return MOE_E_ALIGN;
  const moe_experts& X = layer->experts;
  const int H = X.hidden, I = X.inter, E = layer->n_experts, k = layer->top_k;
  const bool shared = layer->shared_slot >= 0;
  const PrefillWs pw = PrefillWs::make(T, H, I, E, k, shared);
  if (!ws || ws_bytes < pw.total) return MOE_E_WORKSPACE;
  uint8_t* w8 = reinterpret_cast<uint8_t*>(ws);
  auto F = [&](size_t o) { return reinterpret_cast<float*>(w8 + o); };
  auto I32 = [&](size_t o) { return reinterpret_cast<int32_t*>(w8 + o); };
  auto F16 = [&](size_t o) { return reinterpret_cast<_Float16*>(w8 + o); };
  const uint8_t* base = reinterpret_cast<const uint8_t*>(X.base);

  hipLaunchKernelGGL(prep_x_kernel, dim3(T), dim3(256), 0, stream, x, H, layer->w_sg,
                     F16(pw.xh), F16(pw.xl), F(pw.xs), F(pw.sglogit));
  const int ks = router_ksplit(T, E, H);
  hipLaunchKernelGGL(router_gemm_kernel, dim3((T + 63) / 64, E / 64, ks), dim3(512), 0, stream, x,
                     T, H, layer->w_router, E, H / ks, F(pw.logits), F(pw.rpart));
  {
    const dim3 rg((T * E + 255) / 256);
    switch (ks) {
      case 1: break;
      case 2: hipLaunchKernelGGL(router_reduce_kernel<2>, rg, dim3(256), 0, stream, F(pw.rpart), T * E, F(pw.logits)); break;
      case 4: hipLaunchKernelGGL(router_reduce_kernel<4>, rg, dim3(256), 0, stream, F(pw.rpart), T * E, F(pw.logits)); break;
      case 8: hipLaunchKernelGGL(router_reduce_kernel<8>, rg, dim3(256), 0, stream, F(pw.rpart), T * E, F(pw.logits)); break;
      case 16: hipLaunchKernelGGL(router_reduce_kernel<16>, rg, dim3(256), 0, stream, F(pw.rpart), T * E, F(pw.logits)); break;
      default: hipLaunchKernelGGL(router_reduce_kernel<32>, rg, dim3(256), 0, stream, F(pw.rpart), T * E, F(pw.logits)); break;
    }
  }
  hipLaunchKernelGGL(prefill_topk_kernel, dim3(T), dim3(64), 0, stream, F(pw.logits), E, k,
                     layer->w_sg ? F(pw.sglogit) : nullptr, I32(pw.ids), F(pw.wts), F(pw.sg),
                     ids_out, weights_out, sg_out);
  hipLaunchKernelGGL(sort_kernel, dim3(1), dim3(1024), 0, stream, I32(pw.ids), T, k, E,
                     layer->shared_slot, I32(pw.a_row), I32(pw.inv),
                     reinterpret_cast<Seg*>(w8 + pw.segs), I32(pw.nseg));
  // one-dimensional grids in the XCD-aware order the kernels decode (segments padded to 8)
  const int seg8 = (pw.max_segs + 7) / 8 * 8;
  // fewer than 64 tokens: one tile per gate/up and down wave, twice the blocks per segment
  const bool gu_fine = T < 64;
  const dim3 gu_grid(seg8 * (I / (gu_fine ? kGuChunk / 2 : kGuChunk))), dn_grid(seg8 * (H / (kDnChunk / 2)));
  const Seg* segs = reinterpret_cast<const Seg*>(w8 + pw.segs);
#define MOE_GU(HH, NTW)                                                                        \
  hipLaunchKernelGGL((gu_grouped_kernel<HH, NTW>), gu_grid, dim3(512), 0, stream, segs,        \
                     I32(pw.nseg), base, X.slot_bytes, I, I32(pw.a_row), F16(pw.xh),           \
                     F16(pw.xl), F(pw.xs), F(pw.hf))
  switch (H) {
    case 1024: if (gu_fine) MOE_GU(1024, 1); else MOE_GU(1024, 2); break;
    case 2048: if (gu_fine) MOE_GU(2048, 1); else MOE_GU(2048, 2); break;
    default: if (gu_fine) MOE_GU(4096, 1); else MOE_GU(4096, 2); break;
  }
#undef MOE_GU
  const size_t n8 = (size_t)pw.rows * I / 8;
  hipLaunchKernelGGL(prep_h_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream,
                     F(pw.hf), pw.rows, I, F16(pw.hh), F16(pw.hl), F(pw.hs));
#define MOE_DN(II, NTW)                                                                        \
  hipLaunchKernelGGL((dn_grouped_kernel<II, NTW>), dn_grid, dim3(512), 0, stream, segs,        \
                     I32(pw.nseg), base, X.slot_bytes, H, F16(pw.hh), F16(pw.hl), F(pw.hs),     \
                     F(pw.y))
  switch (I) {
    case 256: MOE_DN(256, 1); break;
    case 512: MOE_DN(512, 1); break;
    case 1024: MOE_DN(1024, 1); break;
    default: MOE_DN(2048, 1); break;
  }
#undef MOE_DN
  hipLaunchKernelGGL(prefill_combine_kernel, dim3((H / 4 + 255) / 256, T), dim3(256), 0, stream,
                     x, T, H, k, F(pw.wts), I32(pw.inv), F(pw.sg), shared ? 1 : 0, F(pw.y), out);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_HIP;
}

}  // extern "C"
