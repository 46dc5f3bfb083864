// moe_decode.hip -- single-token (decode) kernels and C entry points of libmoe.
//
// One MoE layer for one token is three kernels on one stream (one HIP-graph chain):
//   K1  router rows (E x H fp32) and the shared expert's gate/up rows with SwiGLU;
//       both depend only on the layer input.
//   K2  top-k of the router logits, recomputed by every wave from the logits K1
//       wrote, then the routed experts' gate/up rows with SwiGLU (a2a-mcp.org "What
//       is Flash-MoE", deep dive 3: fused SwiGLU).
//   K3  down rows of the k routed + shared experts, with the weighted combine, the
//       sigmoid-gated shared expert and the residual add done in the same block
//       (deep dive 3: combine + residual + gating in one pass).
// The routing decision never leaves the device (the wiki summary's per-layer
// pipeline hands the expert work to the GPU without a host round trip).  No kernel
// uses atomics or cross-block waits: every dependency is a kernel boundary, and the
// values several blocks need (top-k, RMS statistics) are recomputed by each of them
// in the same order, so they agree bitwise.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"
#include "moe_device.h"
#include "moe_host.h"
#include "moe_persist.h"

namespace moe {
namespace {

constexpr int kBlock = 512;  // threads of K1/K2 blocks (8 waves)

// x [H] staged in LDS by the whole block: load into registers first (issued before the
// weight loads, so waiting for x does not wait for the weights), then store.
template <int H>
__device__ __forceinline__ void xstage_load(const float* __restrict__ x, float4& v0, float4& v1) {
  static_assert(H / 4 <= 2 * 512, "at most two float4 per thread");
  const float4* s4 = reinterpret_cast<const float4*>(x);
  const int i = threadIdx.x;
  if (H / 4 >= 512 || i < H / 4) v0 = s4[i];
  if (H / 4 > 512) v1 = s4[i + 512];
}
template <int H>
__device__ __forceinline__ void xstage_store(float* xs, const float4& v0, const float4& v1) {
  float4* d4 = reinterpret_cast<float4*>(xs);
  const int i = threadIdx.x;
  if (H / 4 >= 512 || i < H / 4) d4[i] = v0;
  if (H / 4 > 512) d4[i + 512] = v1;
}

// 1/sqrt(mean(x^2) + eps) from a wave whose lanes jointly hold all of x in lr.x.
template <int BITS, int H>
__device__ __forceinline__ float rms_scale_from(const LaneRow<BITS, H>& lr, float eps) {
  using G = Geo<BITS, H>;
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < G::kXPerLane; ++i) ss = fmaf(lr.x[i], lr.x[i], ss);
  ss = seg_sum<G::kLanesPerRow>(ss);
  return 1.f / sqrtf(ss / (float)H + eps);
}

// ------------------------------------------------------------------------------------------
// K1: router logits + shared-expert gate/up/SwiGLU.
// Block b: router rows 2b, 2b+1 (one quarter row per wave) and h rows 4b..4b+3 of the
// shared expert (waves 0-3 gate rows, waves 4-7 up rows).  grid.y = token (router only).
// ------------------------------------------------------------------------------------------
struct K1Args {
  const float* x;         // [T][H]
  int norm;               // inputs are RMSNorm(x) (scale recomputed from x)
  float eps;
  const float* w_router;  // [E][H] or null
  int E;
  float* logits;          // [T][E]
  const uint8_t* shared;  // shared expert record or null (T must be 1)
  int I;
  float* h_shared;        // [I]
};

template <int BITS, int H, bool SHARED>
__global__ __launch_bounds__(kBlock) void k1_kernel(K1Args a) {
  using G = Geo<BITS, H>;
  constexpr int kQ = H / 4 / 4 / 64;  // float4 per lane in a quarter row
  __shared__ float xs[H];
  __shared__ float part[8];
  __shared__ float gbuf[4];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.y;

  float4 xv0, xv1;
  xstage_load<H>(a.x + (size_t)t * H, xv0, xv1);
  issue_fence();
  // router quarter row r (4 waves per row); rows past E load row E-1 and are not written
  const int r = blockIdx.x * 2 + (wave >> 2);
  const int q = wave & 3;
  const bool do_router = r < a.E;
  float4 wv[kQ];
  {
    const float* wr = a.w_router + (size_t)(do_router ? r : a.E - 1) * H + q * (H / 4);
#pragma unroll
    for (int j = 0; j < kQ; ++j) wv[j] = ld_nt_f4(wr + 4 * (lane + 64 * j));
  }
  // shared expert: gate (waves 0-3) or up (waves 4-7) row hi
  const int hi = blockIdx.x * 4 + (wave & 3);
  const bool do_shared = SHARED && hi < a.I;
  LaneRow<BITS, H> lr;
  lr.set_lane(lane);
  RowLoad<BITS, H> ld;
  if constexpr (SHARED) {
    const size_t mat = matrix_rec_bytes<BITS>(a.I, H);
    ld.load(a.shared + (wave < 4 ? 0 : mat), a.I, do_shared ? hi : a.I - 1, lr);
  }
  issue_fence();
  xstage_store<H>(xs, xv0, xv1);
  __syncthreads();
  lr.load_x(xs);
  lr.finish();
  const float xscale = a.norm ? rms_scale_from<BITS, H>(lr, a.eps) : 1.f;

  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < kQ; ++j) {
    const float4 xq = reinterpret_cast<const float4*>(xs + q * (H / 4))[lane + 64 * j];
    acc = fmaf(wv[j].x, xq.x, acc);
    acc = fmaf(wv[j].y, xq.y, acc);
    acc = fmaf(wv[j].z, xq.z, acc);
    acc = fmaf(wv[j].w, xq.w, acc);
  }
  acc = seg_sum<64>(acc);
  if (lane == 0) part[wave] = acc;
  float gu = 0.f;
  if constexpr (SHARED) {
    gu = seg_sum<G::kLanesPerRow>(ld.partial(lr)) * xscale;
    if (wave < 4 && lane == 0) gbuf[wave] = gu;
  }
  __syncthreads();
  if (do_router && q == 0 && lane == 0)  // waves wave..wave+3 hold the four quarters of row r
    a.logits[(size_t)t * a.E + r] =
        (((part[wave] + part[wave + 1]) + part[wave + 2]) + part[wave + 3]) * xscale;
  if (do_shared && wave >= 4 && lane == 0) a.h_shared[hi] = siluf_acc(gbuf[wave - 4]) * gu;
}

// ------------------------------------------------------------------------------------------
// K2: routed gate/up/SwiGLU.  With R = rows per wave pass, a block covers 16R h rows of one
// slot: wave w handles rows base + 2Rw + sub and base + 2Rw + R + sub (sub = lane's row within
// the pass).  Slot ids come from top-k of the router logits (each wave recomputes it) or from
// an id array.
// ------------------------------------------------------------------------------------------
struct K2Args {
  const float* x;          // [H]
  int norm;
  float eps;
  const float* logits;     // [E]: top-k mode when not null
  int E, k;
  const int32_t* ids_in;   // id mode: [n]
  int n;                   // slots processed (k in top-k mode)
  const uint8_t* base;
  int64_t slot_bytes;
  int n_slots_total;
  int I;
  float* h;                // [n][I]
  // top-k mode: routing outputs written by block 0, wave 0
  int32_t* ids_ws;         // [k+1] (shared slot appended when shared_slot >= 0)
  float* w_ws;             // [k]
  float* sg_ws;            // [1]
  int shared_slot;
  const float* w_sg;       // [H] or null (gate 1)
  int32_t* ids_out;        // optional copies
  float* w_out;
  float* sg_out;
  int32_t* ids_trace;      // optional [k]
  int32_t* dev_err;
};

template <int BITS, int H>
constexpr int k2_rows_per_block() { return 16 * Geo<BITS, H>::kRowsPerWave; }

template <int BITS, int H>
__global__ __launch_bounds__(kBlock) void k2_kernel(K2Args a) {
  using G = Geo<BITS, H>;
  constexpr int R = G::kRowsPerWave;
  __shared__ float xs[H];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int blocks_per_slot = a.I / k2_rows_per_block<BITS, H>();
  const int j = blockIdx.x / blocks_per_slot;
  float4 xv0, xv1;
  xstage_load<H>(a.x, xv0, xv1);
  LaneRow<BITS, H> lr;
  lr.set_lane(lane);
  const int i0 = (blockIdx.x % blocks_per_slot) * k2_rows_per_block<BITS, H>() + 2 * R * wave +
                 lr.sub;
  const int i1 = i0 + R;

  int ids[kMaxTopK];
  float vals[kMaxTopK], w[kMaxTopK];
  int e;
  if (a.logits) {
    wave_topk(a.logits, a.E, a.k, ids, vals, w);
    e = ids[0];
#pragma unroll
    for (int s = 1; s < kMaxTopK; ++s)
      if (s == j) e = ids[s];
  } else {
    e = a.ids_in[j];
  }
  const bool valid = e >= 0 && e < a.n_slots_total;  // invalid ids load slot 0, write zeros
  RowLoad<BITS, H> lg0, lg1, lu0, lu1;
  const size_t mat = matrix_rec_bytes<BITS>(a.I, H);
  {
    const uint8_t* rec = a.base + (size_t)(valid ? e : 0) * a.slot_bytes;
    lg0.load(rec, a.I, i0, lr);
    lg1.load(rec, a.I, i1, lr);
    lu0.load(rec + mat, a.I, i0, lr);
    lu1.load(rec + mat, a.I, i1, lr);
  }
  issue_fence();
  xstage_store<H>(xs, xv0, xv1);
  __syncthreads();
  lr.load_x(xs);
  lr.finish();
  const float xscale = a.norm ? rms_scale_from<BITS, H>(lr, a.eps) : 1.f;

  if (a.logits && blockIdx.x == 0 && wave == 0) {
    // routing outputs for K3 (and the optional copies)
    float sgv = 1.f;
    if (a.w_sg) {
      float acc = 0.f;
#pragma unroll
      for (int p = 0; p < G::kPasses; ++p) {
        const float* ws = a.w_sg + lr.chunk[p] * G::kCodesPerChunk;
#pragma unroll
        for (int c = 0; c < G::kCodesPerChunk; ++c)
          acc = fmaf(ws[c], lr.x[p * G::kCodesPerChunk + c], acc);
      }
      sgv = sigmoidf_acc(seg_sum<G::kLanesPerRow>(acc) * xscale);
    }
    if (lane == 0) {
#pragma unroll
      for (int s = 0; s < kMaxTopK; ++s) {
        if (s >= a.k) break;
        a.ids_ws[s] = ids[s];
        a.w_ws[s] = w[s];
        if (a.ids_out) a.ids_out[s] = ids[s];
        if (a.w_out) a.w_out[s] = w[s];
        if (a.ids_trace) a.ids_trace[s] = ids[s];
      }
      if (a.shared_slot >= 0) {
        a.ids_ws[a.k] = a.shared_slot;
        if (a.ids_out) a.ids_out[a.k] = a.shared_slot;
      }
      *a.sg_ws = sgv;
      if (a.sg_out) *a.sg_out = sgv;
    }
  }

  float g0 = lg0.partial(lr);
  float g1 = lg1.partial(lr);
  float u0 = lu0.partial(lr);
  float u1 = lu1.partial(lr);
  g0 = seg_sum<G::kLanesPerRow>(g0) * xscale;
  g1 = seg_sum<G::kLanesPerRow>(g1) * xscale;
  u0 = seg_sum<G::kLanesPerRow>(u0) * xscale;
  u1 = seg_sum<G::kLanesPerRow>(u1) * xscale;
  if ((lane % G::kLanesPerRow) == 0) {
    float* hj = a.h + (size_t)j * a.I;
    hj[i0] = valid ? siluf_acc(g0) * u0 : 0.f;
    hj[i1] = valid ? siluf_acc(g1) * u1 : 0.f;
  }
  if (!valid && lane == 0 && a.dev_err) *a.dev_err = 1;
}

// ------------------------------------------------------------------------------------------
// K3: down rows for n slots over kDownRows output rows per block; wave j handles slot j.
// Mode Y (y != null): y[j][r] = deq(W_down[ids[j]]) h[j].
// Mode combine: out[r] = residual[r] + sum_j coef_j * y_j[r], coef_j = route_w[j] for
// j < n_routed, else *sg (or 1 when sg is null).
// ------------------------------------------------------------------------------------------
struct K3Args {
  const uint8_t* base;
  int64_t slot_bytes;
  int n_slots_total;
  const int32_t* ids;
  int n;
  const float* h;        // [n][I]
  int H;
  float* y;              // mode Y
  const float* residual;
  const float* route_w;
  int n_routed;
  const float* sg;
  float* out;
  int32_t* dev_err;
};

template <int BITS, int I>
__global__ __launch_bounds__(512) void k3_kernel(K3Args a) {
  using G = Geo<BITS, I>;
  constexpr int kRB = kDownRows / G::kRowsPerWave;  // row blocks per wave
  static_assert(kDownRows % G::kRowsPerWave == 0, "");
  const int lane = threadIdx.x & 63;
  const int j = threadIdx.x >> 6;
  const int r0 = blockIdx.x * kDownRows;
  __shared__ float ybuf[8][kDownRows];

  const int e = a.ids[j];
  const bool valid = e >= 0 && e < a.n_slots_total;
  LaneRow<BITS, I> lr;
  lr.set_lane(lane);
  lr.load_x(a.h + (size_t)j * I);
  issue_fence();
  RowLoad<BITS, I> ld[kRB];
  {
    // invalid ids load slot 0 and contribute zeros
    const uint8_t* rec = a.base + (size_t)(valid ? e : 0) * a.slot_bytes +
                         2 * matrix_rec_bytes<BITS>(I, a.H);
#pragma unroll
    for (int b = 0; b < kRB; ++b) ld[b].load(rec, a.H, r0 + b * G::kRowsPerWave + lr.sub, lr);
  }
  issue_fence();
  lr.finish();
#pragma unroll
  for (int b = 0; b < kRB; ++b) {
    const float v = seg_sum<G::kLanesPerRow>(ld[b].partial(lr));
    if ((lane % G::kLanesPerRow) == 0) ybuf[j][b * G::kRowsPerWave + lr.sub] = valid ? v : 0.f;
  }
  if (!valid && lane == 0 && a.dev_err) *a.dev_err = 1;
  __syncthreads();
  if (a.y) {
    for (int i = threadIdx.x; i < a.n * kDownRows; i += blockDim.x) {
      const int jj = i / kDownRows, rr = i % kDownRows;
      a.y[(size_t)jj * a.H + r0 + rr] = ybuf[jj][rr];
    }
    return;
  }
  if (threadIdx.x < kDownRows) {
    const int r = r0 + threadIdx.x;
    float o = a.residual[r];
    for (int jj = 0; jj < a.n; ++jj) {
      const float c = jj < a.n_routed ? a.route_w[jj] : (a.sg ? *a.sg : 1.f);
      o = fmaf(c, ybuf[jj][threadIdx.x], o);
    }
    a.out[r] = o;
  }
}

// xn = x / sqrt(mean(x^2) + eps), one block per row of H (row blockIdx.x).  Each thread
// writes only the elements it read, after the block-wide sum, so xn may equal x.
__global__ __launch_bounds__(1024) void rmsnorm_kernel(const float* x, int H, float eps,
                                                      float* xn) {
  __shared__ float red[16];
  x += (size_t)blockIdx.x * H;
  xn += (size_t)blockIdx.x * H;
  constexpr int kKeep = 8;  // the first 8 * blockDim.x elements stay in registers
  float v[kKeep];
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kKeep; ++j) {
    const int i = threadIdx.x + j * blockDim.x;
    v[j] = i < H ? x[i] : 0.f;
  }
#pragma unroll
  for (int j = 0; j < kKeep; ++j) s = fmaf(v[j], v[j], s);
  for (int i = threadIdx.x + kKeep * blockDim.x; i < H; i += blockDim.x) s = fmaf(x[i], x[i], s);
  s = block_sum(s, red);
  const float sc = 1.f / sqrtf(s / (float)H + eps);
#pragma unroll
  for (int j = 0; j < kKeep; ++j) {
    const int i = threadIdx.x + j * blockDim.x;
    if (i < H) xn[i] = v[j] * sc;
  }
  for (int i = threadIdx.x + kKeep * blockDim.x; i < H; i += blockDim.x) xn[i] = x[i] * sc;
}

// Router top-k for T tokens, one wave per token (router_topk entry point).
__global__ __launch_bounds__(64) void topk_kernel(const float* __restrict__ logits, int E, int k,
                                                  const float* __restrict__ x,
                                                  const float* __restrict__ w_sg, int H,
                                                  int32_t* ids, int ld_ids, float* weights,
                                                  float* sg) {
  const int t = blockIdx.x;
  int id[kMaxTopK];
  float vals[kMaxTopK], w[kMaxTopK];
  wave_topk(logits + (size_t)t * E, E, k, id, vals, w);
  float g = 0.f;
  if (w_sg && sg) {
    for (int c = threadIdx.x; c < H; c += 64) g = fmaf(w_sg[c], x[(size_t)t * H + c], g);
    g = sigmoidf_acc(seg_sum<64>(g));
  }
  if (threadIdx.x == 0) {
    for (int s = 0; s < k; ++s) {
      ids[(size_t)t * ld_ids + s] = id[s];
      weights[(size_t)t * k + s] = w[s];
    }
    if (w_sg && sg) sg[t] = g;
  }
}

// ------------------------------------------------------------------------------------------
// Generic quantized matvec y = deq(W) x (building block export).
// ------------------------------------------------------------------------------------------
template <int BITS, int C>
__global__ __launch_bounds__(256) void qgemv_kernel(const uint8_t* __restrict__ rec, int R,
                                                    const float* __restrict__ x,
                                                    float* __restrict__ y) {
  using G = Geo<BITS, C>;
  constexpr int U = 4;
  // x is staged once per workgroup: every wave needs all of it, and reading it from global
  // memory per wave costs more L1 misses than the wave's own weight rows at C = 8192.  Each
  // chunk's inputs are followed by 4 pad floats so that lanes reading consecutive chunks
  // start on different LDS banks.
  constexpr int kStride = G::kCodesPerChunk + 4;
  __shared__ __align__(16) float xs[G::kChunksPerRow * kStride];
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * (blockDim.x >> 6);
  LaneRow<BITS, C> lr;
  lr.set_lane(lane);
  const int nrb = (R + G::kRowsPerWave - 1) / G::kRowsPerWave;
  RowLoad<BITS, C> ld[U];
  int row[U];
  auto issue = [&](int b0) {
#pragma unroll
    for (int i = 0; i < U; ++i) {
      row[i] = (b0 + i) * G::kRowsPerWave + lr.sub;
      if (b0 + i < nrb && row[i] < R) ld[i].load(rec, R, row[i], lr);
    }
  };
  int b0 = wave * U;
  issue(b0);  // the first rows are in flight while x is staged
  for (int i = threadIdx.x; i < C / 4; i += blockDim.x) {
    const float4 v = reinterpret_cast<const float4*>(x)[i];
    const int c = 4 * i;
    *reinterpret_cast<float4*>(&xs[(c / G::kCodesPerChunk) * kStride + c % G::kCodesPerChunk]) = v;
  }
  __syncthreads();
  lr.load_x(xs, kStride);
  lr.finish();
  for (; b0 < nrb; b0 += nwaves * U) {
#pragma unroll
    for (int i = 0; i < U; ++i) {
      if (b0 + i >= nrb) break;
      const bool ok = row[i] < R;
      float v = seg_sum<G::kLanesPerRow>(ok ? ld[i].partial(lr) : 0.f);
      if (ok && (lane % G::kLanesPerRow) == 0) y[row[i]] = v;
    }
    if (b0 + nwaves * U < nrb) issue(b0 + nwaves * U);
  }
}

// Standalone combine (one block) with optional two-pass RMSNorm.
__global__ __launch_bounds__(1024) void combine_kernel(const float* __restrict__ residual,
                                                       const float* __restrict__ y,
                                                       const float* __restrict__ w, int k,
                                                       const float* __restrict__ sg,
                                                       float* out, float* __restrict__ out_norm,
                                                       float eps, int H) {
  __shared__ float red[16];
  const float g = sg ? *sg : 1.f;
  float ss = 0.f;
  for (int c = threadIdx.x; c < H; c += blockDim.x) {
    float o = residual[c];
    for (int j = 0; j < k; ++j) o = fmaf(w[j], y[(size_t)j * H + c], o);
    o = fmaf(g, y[(size_t)k * H + c], o);
    out[c] = o;
    ss = fmaf(o, o, ss);
  }
  if (!out_norm) return;
  ss = block_sum(ss, red);
  const float xs = 1.f / sqrtf(ss / (float)H + eps);
  for (int c = threadIdx.x; c < H; c += blockDim.x) out_norm[c] = out[c] * xs;
}

// strided record copy, 16 bytes per thread step
__global__ void pack_kernel(const uint4* __restrict__ src, int64_t src_stride16, uint4* dst,
                            int64_t dst_stride16, int64_t rec16, int n) {
  const int64_t total = rec16 * n;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t s = i / rec16, o = i - s * rec16;
    dst[s * dst_stride16 + o] = src[s * src_stride16 + o];
  }
}

// column-blocked router copy: dst[c][e][0..15] = src[e][16 c .. 16 c + 15], one 64-byte
// segment per thread
__global__ void pack_router_kernel(const float4* __restrict__ src, int n_experts, int hidden,
                                   float4* __restrict__ dst) {
  const int64_t nseg = (int64_t)n_experts * (hidden / 16);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nseg;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t c = i / n_experts, e = i - c * n_experts;  // dst order: block c, expert e
    const float4* s = src + (e * hidden + 16 * c) / 4;
    float4* d = dst + 4 * i;
#pragma unroll
    for (int k = 0; k < 4; ++k) d[k] = s[k];
  }
}

// ------------------------------------------------------------------------------------------
// launch helpers (template dispatch over the supported shapes)
// ------------------------------------------------------------------------------------------
inline moe_status last_error() { return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_HIP; }

template <int BITS, bool SHARED>
void launch_k1_bs(const K1Args& a, int H, dim3 grid, hipStream_t s) {
  switch (H) {
    case 1024: hipLaunchKernelGGL((k1_kernel<BITS, 1024, SHARED>), grid, dim3(kBlock), 0, s, a); break;
    case 2048: hipLaunchKernelGGL((k1_kernel<BITS, 2048, SHARED>), grid, dim3(kBlock), 0, s, a); break;
    default: hipLaunchKernelGGL((k1_kernel<BITS, 4096, SHARED>), grid, dim3(kBlock), 0, s, a); break;
  }
}
// router rows for T tokens; with a shared expert (T == 1) also its gate/up rows
void launch_k1(const K1Args& a, int bits, int H, int T, hipStream_t s) {
  const int rb = (a.E + 1) / 2;
  const int sb = a.shared ? a.I / 4 : 0;
  const dim3 grid(rb > sb ? rb : sb, T);
  if (!a.shared)
    launch_k1_bs<4, false>(a, H, grid, s);
  else if (bits == 4)
    launch_k1_bs<4, true>(a, H, grid, s);
  else
    launch_k1_bs<2, true>(a, H, grid, s);
}

template <int BITS>
void launch_k2_b(const K2Args& a, int H, hipStream_t s) {
  switch (H) {
    case 1024:
      hipLaunchKernelGGL((k2_kernel<BITS, 1024>), dim3(a.n * (a.I / k2_rows_per_block<BITS, 1024>())),
                         dim3(kBlock), 0, s, a);
      break;
    case 2048:
      hipLaunchKernelGGL((k2_kernel<BITS, 2048>), dim3(a.n * (a.I / k2_rows_per_block<BITS, 2048>())),
                         dim3(kBlock), 0, s, a);
      break;
    default:
      hipLaunchKernelGGL((k2_kernel<BITS, 4096>), dim3(a.n * (a.I / k2_rows_per_block<BITS, 4096>())),
                         dim3(kBlock), 0, s, a);
      break;
  }
}
void launch_k2(const K2Args& a, int bits, int H, hipStream_t s) {
  if (bits == 4) launch_k2_b<4>(a, H, s); else launch_k2_b<2>(a, H, s);
}

template <int BITS>
void launch_k3_b(const K3Args& a, int I, hipStream_t s) {
  dim3 grid(a.H / kDownRows), block(64 * a.n);
  switch (I) {
    case 256: hipLaunchKernelGGL((k3_kernel<BITS, 256>), grid, block, 0, s, a); break;
    case 512: hipLaunchKernelGGL((k3_kernel<BITS, 512>), grid, block, 0, s, a); break;
    case 1024: hipLaunchKernelGGL((k3_kernel<BITS, 1024>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((k3_kernel<BITS, 2048>), grid, block, 0, s, a); break;
  }
}
void launch_k3(const K3Args& a, int bits, int I, hipStream_t s) {
  if (bits == 4) launch_k3_b<4>(a, I, s); else launch_k3_b<2>(a, I, s);
}

template <int BITS>
void launch_qgemv_b(const uint8_t* rec, int R, int C, const float* x, float* y, hipStream_t s) {
  auto grid_for = [&](int rows_per_wave) {
    const int nrb = (R + rows_per_wave - 1) / rows_per_wave;
    const int waves = (nrb + 3) / 4;
    return dim3((waves + 3) / 4);
  };
  switch (C) {
    case 256: hipLaunchKernelGGL((qgemv_kernel<BITS, 256>), grid_for(Geo<BITS, 256>::kRowsPerWave), dim3(256), 0, s, rec, R, x, y); break;
    case 512: hipLaunchKernelGGL((qgemv_kernel<BITS, 512>), grid_for(Geo<BITS, 512>::kRowsPerWave), dim3(256), 0, s, rec, R, x, y); break;
    case 1024: hipLaunchKernelGGL((qgemv_kernel<BITS, 1024>), grid_for(Geo<BITS, 1024>::kRowsPerWave), dim3(256), 0, s, rec, R, x, y); break;
    case 2048: hipLaunchKernelGGL((qgemv_kernel<BITS, 2048>), grid_for(Geo<BITS, 2048>::kRowsPerWave), dim3(256), 0, s, rec, R, x, y); break;
    case 4096: hipLaunchKernelGGL((qgemv_kernel<BITS, 4096>), grid_for(Geo<BITS, 4096>::kRowsPerWave), dim3(256), 0, s, rec, R, x, y); break;
    default: hipLaunchKernelGGL((qgemv_kernel<BITS, 8192>), grid_for(Geo<BITS, 8192>::kRowsPerWave), dim3(256), 0, s, rec, R, x, y); break;
  }
}

// One decode layer on a prepared workspace: K1 -> K2 -> K3.
struct LayerCall {
  const moe_layer* L;
  const float* x;      // residual (layer input)
  int norm;            // router and experts see RMSNorm(x)
  float eps;
  float* out;
  int32_t* ids_out;
  float* weights_out;
  float* sg_out;
  int32_t* ids_trace;
};

moe_status run_layer(const LayerCall& c, uint8_t* ws, const LayerWs& lw, hipStream_t s) {
  const moe_layer* L = c.L;
  const moe_experts& X = L->experts;
  const int H = X.hidden, I = X.inter, E = L->n_experts, k = L->top_k;
  const bool has_shared = L->shared_slot >= 0;
  const int n = k + (has_shared ? 1 : 0);
  const uint8_t* base = reinterpret_cast<const uint8_t*>(X.base);
  float* logits = reinterpret_cast<float*>(ws + lw.logits);
  int32_t* ids = reinterpret_cast<int32_t*>(ws + lw.ids);
  float* weights = reinterpret_cast<float*>(ws + lw.weights);
  float* sg = reinterpret_cast<float*>(ws + lw.sg);
  float* h = reinterpret_cast<float*>(ws + lw.h);

  K1Args a1{};
  a1.x = c.x;
  a1.norm = c.norm;
  a1.eps = c.eps;
  a1.w_router = L->w_router;
  a1.E = E;
  a1.logits = logits;
  a1.shared = has_shared ? base + (size_t)L->shared_slot * X.slot_bytes : nullptr;
  a1.I = I;
  a1.h_shared = h + (size_t)k * I;
  launch_k1(a1, X.bits, H, 1, s);

  K2Args a2{};
  a2.x = c.x;
  a2.norm = c.norm;
  a2.eps = c.eps;
  a2.logits = logits;
  a2.E = E;
  a2.k = k;
  a2.n = k;
  a2.base = base;
  a2.slot_bytes = X.slot_bytes;
  a2.n_slots_total = X.n_slots;
  a2.I = I;
  a2.h = h;
  a2.ids_ws = ids;
  a2.w_ws = weights;
  a2.sg_ws = sg;
  a2.shared_slot = L->shared_slot;
  a2.w_sg = L->w_sg;
  a2.ids_out = c.ids_out;
  a2.w_out = c.weights_out;
  a2.sg_out = c.sg_out;
  a2.ids_trace = c.ids_trace;
  a2.dev_err = X.dev_err;
  launch_k2(a2, X.bits, H, s);

  K3Args a3{};
  a3.base = base;
  a3.slot_bytes = X.slot_bytes;
  a3.n_slots_total = X.n_slots;
  a3.ids = ids;
  a3.n = n;
  a3.h = h;
  a3.H = H;
  a3.y = nullptr;
  a3.residual = c.x;
  a3.route_w = weights;
  a3.n_routed = k;
  a3.sg = sg;
  a3.out = c.out;
  a3.dev_err = X.dev_err;
  launch_k3(a3, X.bits, I, s);
  return last_error();
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_E_NULL: return "required pointer is NULL";
    case MOE_E_SHAPE: return "unsupported or inconsistent shape";
    case MOE_E_ALIGN: return "pointer or stride not 16-byte aligned";
    case MOE_E_BITS: return "bits must be 4 or 2";
    case MOE_E_WORKSPACE: return "workspace missing or too small";
    case MOE_E_HIP: return "HIP launch error";
  }
  return "unknown status";
}

const char* moe_version(void) { return "libmoe 0.2 gfx950"; }

size_t moe_router_workspace_bytes(int T, int E) {
  if (T < 1 || E < 1) return 0;
  return align_up((size_t)T * E * sizeof(float));
}

moe_status moe_router_topk(const float* x, int T, const float* w_router, const float* w_sg,
                           int H, int E, int k, int32_t* ids, int ld_ids, float* weights,
                           float* shared_gate, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!x || !w_router || !ids || !weights) return MOE_E_NULL;
  if (T < 1 || T > 65535 || !hidden_ok(H) || E < 1 || E > 1024 || k < 1 || k > kMaxTopK ||
      k > E || ld_ids < k)
    return MOE_E_SHAPE;
  if (!aligned16(x) || !aligned16(w_router) || (w_sg && !aligned16(w_sg))) return MOE_E_ALIGN;
  if (!ws || ws_bytes < moe_router_workspace_bytes(T, E)) return MOE_E_WORKSPACE;
  float* logits = reinterpret_cast<float*>(ws);
  K1Args a1{};
  a1.x = x;
  a1.norm = 0;
  a1.w_router = w_router;
  a1.E = E;
  a1.logits = logits;
  a1.shared = nullptr;
  a1.I = 4;
  launch_k1(a1, 4, H, T, stream);
  hipLaunchKernelGGL(topk_kernel, dim3(T), dim3(64), 0, stream, logits, E, k, x, w_sg, H, ids,
                     ld_ids, weights, shared_gate);
  return last_error();
}

static moe_status expert_ffn(int bits, const moe_experts* w, const float* x, const int32_t* ids,
                             int n, float* y, float* h, hipStream_t stream) {
  moe_status st = check_experts(w);
  if (st != MOE_OK) return st;
  if (w->bits != bits) return MOE_E_BITS;
  if (!x || !ids || !y || !h) return MOE_E_NULL;
  if (n < 1 || n > 8) return MOE_E_SHAPE;
  if (!aligned16(x) || !aligned16(h)) return MOE_E_ALIGN;
  const uint8_t* base = reinterpret_cast<const uint8_t*>(w->base);
  K2Args a2{};
  a2.x = x;
  a2.norm = 0;
  a2.logits = nullptr;
  a2.ids_in = ids;
  a2.n = n;
  a2.base = base;
  a2.slot_bytes = w->slot_bytes;
  a2.n_slots_total = w->n_slots;
  a2.I = w->inter;
  a2.h = h;
  a2.shared_slot = -1;
  a2.dev_err = w->dev_err;
  launch_k2(a2, bits, w->hidden, stream);
  K3Args a3{};
  a3.base = base;
  a3.slot_bytes = w->slot_bytes;
  a3.n_slots_total = w->n_slots;
  a3.ids = ids;
  a3.n = n;
  a3.h = h;
  a3.H = w->hidden;
  a3.y = y;
  a3.dev_err = w->dev_err;
  launch_k3(a3, bits, w->inter, stream);
  return last_error();
}

moe_status moe_expert_ffn_q4(const moe_experts* w, const float* x, const int32_t* ids, int n,
                             float* y, float* h, hipStream_t stream) {
  return expert_ffn(4, w, x, ids, n, y, h, stream);
}

moe_status moe_expert_ffn_q2(const moe_experts* w, const float* x, const int32_t* ids, int n,
                             float* y, float* h, hipStream_t stream) {
  return expert_ffn(2, w, x, ids, n, y, h, stream);
}

moe_status moe_combine(const float* residual, const float* y, const float* weights, int k,
                       const float* shared_gate, float* out, float* out_norm, float eps, int H,
                       hipStream_t stream) {
  if (!residual || !y || !weights || !out) return MOE_E_NULL;
  if (k < 0 || k > kMaxTopK || H < 1) return MOE_E_SHAPE;
  hipLaunchKernelGGL(combine_kernel, dim3(1), dim3(1024), 0, stream, residual, y, weights, k,
                     shared_gate, out, out_norm, eps, H);
  return last_error();
}

size_t moe_layer_workspace_bytes(const moe_layer* layer) {
  if (check_layer(layer) != MOE_OK) return 0;
  return LayerWs::make(layer->experts.hidden, layer->experts.inter, layer->n_experts,
                       layer->top_k, false).total;
}

moe_status moe_layer_decode(const moe_layer* layer, const float* x, int norm_input, float eps,
                            float* out, int32_t* ids_out, float* weights_out, float* sg_out,
                            void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_layer(layer);
  if (st != MOE_OK) return st;
  if (!x || !out) return MOE_E_NULL;
  if (!aligned16(x) || !aligned16(out)) return MOE_E_ALIGN;
  if (x == out) return MOE_E_SHAPE;
  const LayerWs lw = LayerWs::make(layer->experts.hidden, layer->experts.inter,
                                   layer->n_experts, layer->top_k, false);
  if (!ws || ws_bytes < lw.total) return MOE_E_WORKSPACE;
  LayerCall c{};
  c.L = layer;
  c.x = x;
  c.norm = norm_input ? 1 : 0;
  c.eps = eps;
  c.out = out;
  c.ids_out = ids_out;
  c.weights_out = weights_out;
  c.sg_out = sg_out;
  return run_layer(c, reinterpret_cast<uint8_t*>(ws), lw, stream);
}

size_t moe_stack_workspace_bytes(const moe_layer* layers, int n_layers) {
  if (!layers || n_layers < 1 || check_layer(&layers[0]) != MOE_OK) return 0;
  return LayerWs::make(layers[0].experts.hidden, layers[0].experts.inter, layers[0].n_experts,
                       layers[0].top_k, true).total +
         align_up(PersistWs::bytes());
}

static int g_stack_mode = MOE_STACK_AUTO;

void moe_set_stack_mode(int mode) {
  __atomic_store_n(&g_stack_mode, mode, __ATOMIC_RELAXED);
}

moe_status moe_decode_stack(const moe_layer* layers, int n_layers, const float* x_in,
                            float* x_out, float* xn_out, float eps, int32_t* ids_trace,
                            void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!layers || !x_in || !x_out) return MOE_E_NULL;
  if (n_layers < 1) return MOE_E_SHAPE;
  for (int l = 0; l < n_layers; ++l) {
    moe_status st = check_layer(&layers[l]);
    if (st != MOE_OK) return st;
    const moe_layer& a = layers[l];
    const moe_layer& b = layers[0];
    if (a.experts.hidden != b.experts.hidden || a.experts.inter != b.experts.inter ||
        a.experts.bits != b.experts.bits || a.n_experts != b.n_experts || a.top_k != b.top_k ||
        (a.shared_slot >= 0) != (b.shared_slot >= 0))
      return MOE_E_SHAPE;
  }
  if (!aligned16(x_in) || !aligned16(x_out) || (xn_out && !aligned16(xn_out)))
    return MOE_E_ALIGN;
  if (x_in == x_out || xn_out == x_out) return MOE_E_SHAPE;
  const int H = layers[0].experts.hidden;
  const LayerWs lw = LayerWs::make(H, layers[0].experts.inter, layers[0].n_experts,
                                   layers[0].top_k, true);
  if (!ws || ws_bytes < lw.total) return MOE_E_WORKSPACE;
  if (ws_bytes < lw.total + align_up(PersistWs::bytes())) return MOE_E_WORKSPACE;
  uint8_t* w8 = reinterpret_cast<uint8_t*>(ws);
  float* xbuf = reinterpret_cast<float*>(w8 + lw.xbuf);
  const int k = layers[0].top_k;
  const int mode = __atomic_load_n(&g_stack_mode, __ATOMIC_RELAXED);
  const bool persist = mode != MOE_STACK_KERNELS && persist_shape_ok(layers, n_layers) &&
                       persist_device_ok();
  if (mode == MOE_STACK_PERSISTENT && !persist) return MOE_E_SHAPE;
  if (persist) {
    // chunks of at most kPersistMaxLayers layers; raw x passes between chunks through xbuf
    for (int l0 = 0, c = 0; l0 < n_layers; l0 += kPersistMaxLayers, ++c) {
      const int nl = n_layers - l0 < kPersistMaxLayers ? n_layers - l0 : kPersistMaxLayers;
      const bool last = l0 + nl == n_layers;
      const float* xi = l0 == 0 ? x_in : xbuf + (size_t)((c - 1) & 1) * H;
      float* xo = last ? x_out : xbuf + (size_t)(c & 1) * H;
      moe_status st = persist_launch(layers + l0, nl, xi, xo, last ? xn_out : nullptr, eps,
                                     ids_trace ? ids_trace + (size_t)l0 * k : nullptr,
                                     w8 + lw.total, stream);
      if (st != MOE_OK) return st;
    }
    return last_error();
  }
  for (int l = 0; l < n_layers; ++l) {
    LayerCall c{};
    c.L = &layers[l];
    c.x = l == 0 ? x_in : xbuf + (size_t)((l - 1) & 1) * H;
    c.out = l == n_layers - 1 ? x_out : xbuf + (size_t)(l & 1) * H;
    c.norm = 1;
    c.eps = eps;
    c.ids_trace = ids_trace ? ids_trace + (size_t)l * k : nullptr;
    moe_status st = run_layer(c, w8, lw, stream);
    if (st != MOE_OK) return st;
  }
  if (xn_out) hipLaunchKernelGGL(rmsnorm_kernel, dim3(1), dim3(1024), 0, stream, x_out, H, eps, xn_out);
  return last_error();
}

moe_status moe_qgemv(const moe_qmatrix* m, const float* x, float* y, hipStream_t stream) {
  if (!m || !m->rec || !x || !y) return MOE_E_NULL;
  if (m->bits != 4 && m->bits != 2) return MOE_E_BITS;
  if (m->group != 64 || m->rows < 1 ||
      !(m->cols == 256 || m->cols == 512 || m->cols == 1024 || m->cols == 2048 ||
        m->cols == 4096 || m->cols == 8192))
    return MOE_E_SHAPE;
  if (!aligned16(m->rec) || !aligned16(x)) return MOE_E_ALIGN;
  const uint8_t* rec = reinterpret_cast<const uint8_t*>(m->rec);
  if (m->bits == 4)
    launch_qgemv_b<4>(rec, m->rows, m->cols, x, y, stream);
  else
    launch_qgemv_b<2>(rec, m->rows, m->cols, x, y, stream);
  return last_error();
}

moe_status moe_rmsnorm(const float* x, int T, int H, float eps, float* out,
                       hipStream_t stream) {
  if (!x || !out) return MOE_E_NULL;
  if (T < 1 || H < 1) return MOE_E_SHAPE;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(T), dim3(1024), 0, stream, x, H, eps, out);
  return last_error();
}

moe_status moe_pack(const void* canonical, int n, int slot0, const moe_experts* dst,
                    hipStream_t stream) {
  moe_status st = check_experts(dst);
  if (st != MOE_OK) return st;
  if (!canonical) return MOE_E_NULL;
  if (n < 1 || slot0 < 0 || slot0 + n > dst->n_slots) return MOE_E_SHAPE;
  if (!aligned16(canonical)) return MOE_E_ALIGN;
  const int64_t rec = expert_bytes(dst->bits, dst->hidden, dst->inter);
  if (rec % 16) return MOE_E_ALIGN;
  uint8_t* base = reinterpret_cast<uint8_t*>(const_cast<void*>(dst->base)) +
                  (size_t)slot0 * dst->slot_bytes;
  hipLaunchKernelGGL(pack_kernel, dim3(1024), dim3(256), 0, stream,
                     reinterpret_cast<const uint4*>(canonical), rec / 16,
                     reinterpret_cast<uint4*>(base), dst->slot_bytes / 16, rec / 16, n);
  return last_error();
}

moe_status moe_pack_router(const float* w_router, int n_experts, int hidden, float* dst,
                           hipStream_t stream) {
  if (!w_router || !dst) return MOE_E_NULL;
  if (n_experts < 1 || hidden < 16 || hidden % 16) return MOE_E_SHAPE;
  if (!aligned16(w_router) || !aligned16(dst)) return MOE_E_ALIGN;
  hipLaunchKernelGGL(pack_router_kernel, dim3(1024), dim3(256), 0, stream,
                     reinterpret_cast<const float4*>(w_router), n_experts, hidden,
                     reinterpret_cast<float4*>(dst));
  return last_error();
}

}  // extern "C"
