// moe_decode.hip -- single-token (decode) kernels and C entry points of libmoe.
//
// Per MoE layer and token the work is three dependent streams of weights:
//   router   : E x H fp32 matvec (+ the shared-gate row), then top-k in the last block
//   gate/up  : for k routed experts + the shared expert, two I x H quantized matvecs
//              with SwiGLU applied in registers (a2a-mcp.org "What is Flash-MoE",
//              deep dive 3: fused SwiGLU)
//   down     : for the same experts, one H x I quantized matvec, with the weighted
//              combine + sigmoid-gated shared expert + residual done in the same
//              block (deep dive 3: combine + residual + gating in one pass), and an
//              optional RMSNorm statistics epilogue (the wiki's per-layer pipeline:
//              CMD3 = expert forward + combine + norm).
// The routing decision never leaves the device: the router writes an expert-id
// table that the expert kernels read (the wiki's pipeline encodes the expert
// command buffer without waiting for the GPU; here there is no host round trip
// at all).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"
#include "moe_device.h"
#include "moe_host.h"

namespace moe {
namespace {

// ------------------------------------------------------------------------------------------
// RMS scale: scale = 1 / sqrt(mean(x^2) + eps)   (one block)
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void rms_scale_kernel(const float* __restrict__ x, int H,
                                                        float eps, float* __restrict__ scale) {
  __shared__ float red[16];
  float s = 0.f;
  for (int i = threadIdx.x; i < H; i += blockDim.x) s += x[i] * x[i];
  s = block_sum(s, red);
  if (threadIdx.x == 0) *scale = 1.f / sqrtf(s / (float)H + eps);
}

// ------------------------------------------------------------------------------------------
// Router: logits = W_r (x * xscale), optional shared-gate row, top-k in the last block.
// grid = (ceil(rows / 2), T); 4 waves per block, each wave one half of a row.
// ------------------------------------------------------------------------------------------
struct RouterArgs {
  const float* x;        // [T][H]
  const float* xscale;   // device scalar or null (same scale for all tokens)
  const float* w;        // [E][H]
  const float* wsg;      // [H] or null
  int E, k, T;
  float* logits;         // [T][E+1]
  unsigned* counters;    // [T], zero on entry, zero on exit
  int32_t* ids;          // [T][ld_ids]: k ids, then shared_slot at column k when >= 0
  int ld_ids;
  float* weights;        // [T][k]
  float* sg;             // [T] or null
  int shared_slot;
  int32_t* ids2;         // optional copy of ids (same format, row stride ld_ids2)
  int ld_ids2;
  float* weights2;       // optional copy
  float* sg2;            // optional copy
  int32_t* ids3;         // optional: the k routed ids only
};

template <int H>
__global__ __launch_bounds__(256) void router_kernel(RouterArgs a) {
  constexpr int kF4PerLane = H / 512;  // float4 per lane per half row
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.y;
  const int rows = a.E + (a.wsg ? 1 : 0);
  const int row = blockIdx.x * 2 + (wave >> 1);
  const int half = wave & 1;
  __shared__ float part[4];
  __shared__ int is_last;

  const float sc = a.xscale ? *a.xscale : 1.f;
  const float4* x4 = reinterpret_cast<const float4*>(a.x + (size_t)t * H);
  float acc = 0.f;
  if (row < rows) {
    const float* wrow = row < a.E ? a.w + (size_t)row * H : a.wsg;
    const float4* w4 = reinterpret_cast<const float4*>(wrow);
    float4 wv[kF4PerLane];
#pragma unroll
    for (int j = 0; j < kF4PerLane; ++j) wv[j] = w4[half * (H / 8) + lane + 64 * j];
#pragma unroll
    for (int j = 0; j < kF4PerLane; ++j) {
      const float4 xv = x4[half * (H / 8) + lane + 64 * j];
      acc = fmaf(wv[j].x, xv.x * sc, acc);
      acc = fmaf(wv[j].y, xv.y * sc, acc);
      acc = fmaf(wv[j].z, xv.z * sc, acc);
      acc = fmaf(wv[j].w, xv.w * sc, acc);
    }
  }
  acc = seg_sum<64>(acc);
  if (lane == 0) part[wave] = acc;
  __syncthreads();
  float* logits = a.logits + (size_t)t * (a.E + 1);
  if (threadIdx.x < 2) {
    const int r = blockIdx.x * 2 + threadIdx.x;
    if (r < rows) logits[r] = part[2 * threadIdx.x] + part[2 * threadIdx.x + 1];
  }
  // last block of this token finishes the routing
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = atomicAdd(&a.counters[t], 1u);
    is_last = (prev == gridDim.x - 1);
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  if (wave != 0) return;
  int ids[kMaxTopK];
  float vals[kMaxTopK], w[kMaxTopK];
  wave_topk(logits, a.E, a.k, ids, vals, w);
  if (lane == 0) {
    const float g = a.wsg ? sigmoidf_acc(logits[a.E]) : 1.f;
    int32_t* o1 = a.ids + (size_t)t * a.ld_ids;
    int32_t* o2 = a.ids2 ? a.ids2 + (size_t)t * a.ld_ids2 : nullptr;
    for (int j = 0; j < a.k; ++j) {
      o1[j] = ids[j];
      a.weights[(size_t)t * a.k + j] = w[j];
      if (o2) o2[j] = ids[j];
      if (a.weights2) a.weights2[(size_t)t * a.k + j] = w[j];
      if (a.ids3) a.ids3[(size_t)t * a.k + j] = ids[j];
    }
    if (a.shared_slot >= 0) {
      o1[a.k] = a.shared_slot;
      if (o2) o2[a.k] = a.shared_slot;
    }
    if (a.sg) a.sg[t] = g;
    if (a.sg2) a.sg2[t] = g;
    a.counters[t] = 0u;
  }
}

// ------------------------------------------------------------------------------------------
// Gate/up + SwiGLU for n expert slots: h[j][i] = silu(g_i) * u_i.
// Each wave walks units (slot, row block); U units are loaded before any is reduced.
// ------------------------------------------------------------------------------------------
struct GateUpArgs {
  const uint8_t* base;
  int64_t slot_bytes;
  int n_slots_total;
  const int32_t* ids;    // [n]
  int n;
  const float* x;        // [H]
  const float* xscale;   // device scalar or null
  int I;
  float* h;              // [n][I]
  int32_t* dev_err;
};

template <int BITS, int H, int U>
__global__ __launch_bounds__(256) void gateup_kernel(GateUpArgs a) {
  using G = Geo<BITS, H>;
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * (blockDim.x >> 6);
  LaneRow<BITS, H> lr;
  lr.init(lane, a.x, a.xscale ? *a.xscale : 1.f);
  const int rb_per_slot = a.I / G::kRowsPerWave;
  const int units = a.n * rb_per_slot;
  const size_t mat_bytes = (size_t)a.I * G::kRowBytes + 4 * (size_t)a.I * G::kGroupsPerRow;
  for (int u0 = wave * U; u0 < units; u0 += nwaves * U) {
    RowLoad<BITS, H> lg[U], lu[U];
    int row[U], slot[U];
    bool valid[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int u = u0 + i;
      valid[i] = false;
      slot[i] = 0;
      row[i] = 0;
      if (u < units) {
        slot[i] = u / rb_per_slot;
        row[i] = (u % rb_per_slot) * G::kRowsPerWave + lr.sub;
        const int e = a.ids[slot[i]];
        if (e >= 0 && e < a.n_slots_total) {
          valid[i] = true;
          const uint8_t* rec = a.base + (size_t)e * a.slot_bytes;
          lg[i].load(rec, a.I, row[i], lr);
          lu[i].load(rec + mat_bytes, a.I, row[i], lr);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < U; ++i) {
      if (u0 + i >= units) break;
      float g = valid[i] ? lg[i].partial(lr) : 0.f;
      float u = valid[i] ? lu[i].partial(lr) : 0.f;
      g = seg_sum<G::kLanesPerRow>(g);
      u = seg_sum<G::kLanesPerRow>(u);
      if ((lane % G::kLanesPerRow) == 0)
        a.h[(size_t)slot[i] * a.I + row[i]] = valid[i] ? siluf_acc(g) * u : 0.f;
      if (!valid[i] && lane == 0 && a.dev_err) *a.dev_err = 1;
    }
  }
}

// ------------------------------------------------------------------------------------------
// Down for n slots over kDownRows output rows per block.  Wave j handles slot j.
// Mode Y (y != null): y[j][r] = deq(W_down[ids[j]]) h[j].
// Mode combine: out[r] = residual[r] + sum_j coef_j * y_j[r], coef_j = route_w[j] for
// j < n_routed, else *sg (or 1); then optional RMSNorm statistics (last block writes
// xscale_next = 1/sqrt(mean(out^2)+eps) and out_norm = out * xscale_next).
// ------------------------------------------------------------------------------------------
struct DownArgs {
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
  float* partials;       // [gridDim.x] (norm epilogue)
  unsigned* counter;     // zero on entry, zero on exit (norm epilogue)
  float eps;
  float* xscale_next;    // or null
  float* out_norm;       // or null
  int32_t* dev_err;
};

template <int BITS, int I>
__global__ __launch_bounds__(512) void down_kernel(DownArgs a) {
  using G = Geo<BITS, I>;
  constexpr int kRB = kDownRows / G::kRowsPerWave;  // row blocks per wave
  static_assert(kDownRows % G::kRowsPerWave == 0, "");
  const int lane = threadIdx.x & 63;
  const int j = threadIdx.x >> 6;  // slot handled by this wave
  const int r0 = blockIdx.x * kDownRows;
  __shared__ float ybuf[8][kDownRows];
  __shared__ int is_last;
  __shared__ float red[16];

  const int e = a.ids[j];
  const bool valid = e >= 0 && e < a.n_slots_total;
  LaneRow<BITS, I> lr;
  lr.init(lane, a.h + (size_t)j * I, 1.f);
  if (valid) {
    const uint8_t* rec = a.base + (size_t)e * a.slot_bytes + 2 * (size_t)matrix_rec_bytes<BITS>(I, a.H);
    RowLoad<BITS, I> ld[kRB];
#pragma unroll
    for (int b = 0; b < kRB; ++b) ld[b].load(rec, a.H, r0 + b * G::kRowsPerWave + lr.sub, lr);
#pragma unroll
    for (int b = 0; b < kRB; ++b) {
      float v = seg_sum<G::kLanesPerRow>(ld[b].partial(lr));
      if ((lane % G::kLanesPerRow) == 0) ybuf[j][b * G::kRowsPerWave + lr.sub] = v;
    }
  } else {
    if (lane < kDownRows) ybuf[j][lane] = 0.f;
    if (lane == 0 && a.dev_err) *a.dev_err = 1;
  }
  __syncthreads();
  if (a.y) {
    for (int i = threadIdx.x; i < a.n * kDownRows; i += blockDim.x) {
      const int jj = i / kDownRows, rr = i % kDownRows;
      a.y[(size_t)jj * a.H + r0 + rr] = ybuf[jj][rr];
    }
    return;
  }
  // combine: threads of wave 0 own one output row each
  if (j == 0) {
    float o = 0.f;
    if (lane < kDownRows) {
      const int r = r0 + lane;
      o = a.residual[r];
      for (int jj = 0; jj < a.n; ++jj) {
        const float c = jj < a.n_routed ? a.route_w[jj] : (a.sg ? *a.sg : 1.f);
        o = fmaf(c, ybuf[jj][lane], o);
      }
      a.out[r] = o;
    }
    if (a.partials) {
      const float ss = seg_sum<64>(o * o);
      if (lane == 0) a.partials[blockIdx.x] = ss;
    }
  }
  if (!a.partials) return;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = atomicAdd(a.counter, 1u);
    is_last = (prev == gridDim.x - 1);
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  float s = 0.f;
  for (int i = threadIdx.x; i < (int)gridDim.x; i += blockDim.x) s += a.partials[i];
  s = block_sum(s, red);
  const float xs = 1.f / sqrtf(s / (float)a.H + a.eps);
  if (a.out_norm)
    for (int r = threadIdx.x; r < a.H; r += blockDim.x) a.out_norm[r] = a.out[r] * xs;
  if (threadIdx.x == 0) {
    if (a.xscale_next) *a.xscale_next = xs;
    *a.counter = 0u;
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
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * (blockDim.x >> 6);
  LaneRow<BITS, C> lr;
  lr.init(lane, x, 1.f);
  const int nrb = (R + G::kRowsPerWave - 1) / G::kRowsPerWave;
  for (int b0 = wave * U; b0 < nrb; b0 += nwaves * U) {
    RowLoad<BITS, C> ld[U];
    int row[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      row[i] = (b0 + i) * G::kRowsPerWave + lr.sub;
      if (b0 + i < nrb && row[i] < R) ld[i].load(rec, R, row[i], lr);
    }
#pragma unroll
    for (int i = 0; i < U; ++i) {
      if (b0 + i >= nrb) break;
      const bool ok = row[i] < R;
      float v = seg_sum<G::kLanesPerRow>(ok ? ld[i].partial(lr) : 0.f);
      if (ok && (lane % G::kLanesPerRow) == 0) y[row[i]] = v;
    }
  }
}

// ------------------------------------------------------------------------------------------
// Standalone combine (one block) with optional two-pass RMSNorm.
// ------------------------------------------------------------------------------------------
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
    ss += o * o;
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

// ------------------------------------------------------------------------------------------
// launch helpers
// ------------------------------------------------------------------------------------------
inline moe_status last_error() { return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_HIP; }

void launch_router(const RouterArgs& a, int H, hipStream_t s) {
  const int rows = a.E + (a.wsg ? 1 : 0);
  dim3 grid((rows + 1) / 2, a.T);
  switch (H) {
    case 1024: hipLaunchKernelGGL(router_kernel<1024>, grid, dim3(256), 0, s, a); break;
    case 2048: hipLaunchKernelGGL(router_kernel<2048>, grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL(router_kernel<4096>, grid, dim3(256), 0, s, a); break;
  }
}

template <int BITS>
void launch_gateup_b(const GateUpArgs& a, int H, hipStream_t s) {
  constexpr int U = 2;
  // one unit = one row of gate and up (times rows per wave pass); size the grid so every
  // wave gets U units
  int rows_per_wave;
  switch (H) {
    case 1024: rows_per_wave = Geo<BITS, 1024>::kRowsPerWave; break;
    case 2048: rows_per_wave = Geo<BITS, 2048>::kRowsPerWave; break;
    default: rows_per_wave = Geo<BITS, 4096>::kRowsPerWave; break;
  }
  const int units = a.n * (a.I / rows_per_wave);
  const int waves = (units + U - 1) / U;
  const int blocks = (waves + 3) / 4;
  switch (H) {
    case 1024: hipLaunchKernelGGL((gateup_kernel<BITS, 1024, U>), dim3(blocks), dim3(256), 0, s, a); break;
    case 2048: hipLaunchKernelGGL((gateup_kernel<BITS, 2048, U>), dim3(blocks), dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((gateup_kernel<BITS, 4096, U>), dim3(blocks), dim3(256), 0, s, a); break;
  }
}

void launch_gateup(const GateUpArgs& a, int bits, int H, hipStream_t s) {
  if (bits == 4)
    launch_gateup_b<4>(a, H, s);
  else
    launch_gateup_b<2>(a, H, s);
}

template <int BITS>
void launch_down_b(const DownArgs& a, int I, hipStream_t s) {
  dim3 grid(a.H / kDownRows), block(64 * a.n);
  switch (I) {
    case 256: hipLaunchKernelGGL((down_kernel<BITS, 256>), grid, block, 0, s, a); break;
    case 512: hipLaunchKernelGGL((down_kernel<BITS, 512>), grid, block, 0, s, a); break;
    case 1024: hipLaunchKernelGGL((down_kernel<BITS, 1024>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((down_kernel<BITS, 2048>), grid, block, 0, s, a); break;
  }
}

void launch_down(const DownArgs& a, int bits, int I, hipStream_t s) {
  if (bits == 4)
    launch_down_b<4>(a, I, s);
  else
    launch_down_b<2>(a, I, s);
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
    default: hipLaunchKernelGGL((qgemv_kernel<BITS, 4096>), grid_for(Geo<BITS, 4096>::kRowsPerWave), dim3(256), 0, s, rec, R, x, y); break;
  }
}

// One decode layer on a prepared workspace.  x_in: residual; xscale: device scalar
// applied to x for router + experts (null = 1).  Writes out, and (optionally) the
// RMSNorm statistics of out.
struct LayerCall {
  const moe_layer* L;
  const float* x;
  const float* xscale;
  float* out;
  float* xscale_next;  // norm epilogue target or null
  float* out_norm;     // or null
  float eps;
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
  unsigned* counters = reinterpret_cast<unsigned*>(ws + lw.counters);
  int32_t* ids = reinterpret_cast<int32_t*>(ws + lw.ids);
  float* weights = reinterpret_cast<float*>(ws + lw.weights);
  float* sg = reinterpret_cast<float*>(ws + lw.sg);
  float* h = reinterpret_cast<float*>(ws + lw.h);

  RouterArgs ra{};
  ra.x = c.x;
  ra.xscale = c.xscale;
  ra.w = L->w_router;
  ra.wsg = L->w_sg;
  ra.E = E;
  ra.k = k;
  ra.T = 1;
  ra.logits = reinterpret_cast<float*>(ws + lw.logits);
  ra.counters = counters + 0;
  ra.ids = ids;
  ra.ld_ids = k + 1;
  ra.weights = weights;
  ra.sg = sg;
  ra.shared_slot = L->shared_slot;
  ra.ids2 = c.ids_out;
  ra.ld_ids2 = k + 1;
  ra.weights2 = c.weights_out;
  ra.sg2 = c.sg_out;
  ra.ids3 = c.ids_trace;
  launch_router(ra, H, s);

  GateUpArgs ga{};
  ga.base = reinterpret_cast<const uint8_t*>(X.base);
  ga.slot_bytes = X.slot_bytes;
  ga.n_slots_total = X.n_slots;
  ga.ids = ids;
  ga.n = n;
  ga.x = c.x;
  ga.xscale = c.xscale;
  ga.I = I;
  ga.h = h;
  ga.dev_err = X.dev_err;
  launch_gateup(ga, X.bits, H, s);

  DownArgs da{};
  da.base = ga.base;
  da.slot_bytes = X.slot_bytes;
  da.n_slots_total = X.n_slots;
  da.ids = ids;
  da.n = n;
  da.h = h;
  da.H = H;
  da.y = nullptr;
  da.residual = c.x;
  da.route_w = weights;
  da.n_routed = k;
  da.sg = sg;
  da.out = c.out;
  const bool norm = c.xscale_next || c.out_norm;
  da.partials = norm ? reinterpret_cast<float*>(ws + lw.partials) : nullptr;
  da.counter = counters + 1;
  da.eps = c.eps;
  da.xscale_next = c.xscale_next;
  da.out_norm = c.out_norm;
  da.dev_err = X.dev_err;
  launch_down(da, X.bits, I, s);
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

const char* moe_version(void) { return "libmoe 0.1 gfx950"; }

size_t moe_router_workspace_bytes(int T, int E) {
  if (T < 1 || E < 1) return 0;
  return align_up((size_t)T * sizeof(unsigned)) + align_up((size_t)T * (E + 1) * sizeof(float));
}

moe_status moe_router_topk(const float* x, int T, const float* w_router, const float* w_sg,
                           int H, int E, int k, int32_t* ids, int ld_ids, float* weights,
                           float* shared_gate, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!x || !w_router || !ids || !weights) return MOE_E_NULL;
  if (T < 1 || !hidden_ok(H) || E < 1 || E > 1024 || k < 1 || k > kMaxTopK || k > E ||
      ld_ids < k)
    return MOE_E_SHAPE;
  if (!aligned16(x) || !aligned16(w_router) || (w_sg && !aligned16(w_sg))) return MOE_E_ALIGN;
  if (!ws || ws_bytes < moe_router_workspace_bytes(T, E)) return MOE_E_WORKSPACE;
  uint8_t* w8 = reinterpret_cast<uint8_t*>(ws);
  RouterArgs ra{};
  ra.x = x;
  ra.xscale = nullptr;
  ra.w = w_router;
  ra.wsg = w_sg;
  ra.E = E;
  ra.k = k;
  ra.T = T;
  ra.counters = reinterpret_cast<unsigned*>(w8);
  ra.logits = reinterpret_cast<float*>(w8 + align_up((size_t)T * sizeof(unsigned)));
  ra.ids = ids;
  ra.ld_ids = ld_ids;
  ra.weights = weights;
  ra.sg = w_sg ? shared_gate : nullptr;
  ra.shared_slot = -1;
  launch_router(ra, H, stream);
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
  GateUpArgs ga{};
  ga.base = reinterpret_cast<const uint8_t*>(w->base);
  ga.slot_bytes = w->slot_bytes;
  ga.n_slots_total = w->n_slots;
  ga.ids = ids;
  ga.n = n;
  ga.x = x;
  ga.xscale = nullptr;
  ga.I = w->inter;
  ga.h = h;
  ga.dev_err = w->dev_err;
  launch_gateup(ga, bits, w->hidden, stream);
  DownArgs da{};
  da.base = ga.base;
  da.slot_bytes = w->slot_bytes;
  da.n_slots_total = w->n_slots;
  da.ids = ids;
  da.n = n;
  da.h = h;
  da.H = w->hidden;
  da.y = y;
  da.dev_err = w->dev_err;
  launch_down(da, bits, w->inter, stream);
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
  uint8_t* w8 = reinterpret_cast<uint8_t*>(ws);
  float* xscale = reinterpret_cast<float*>(w8 + lw.xscale);
  if (norm_input)
    hipLaunchKernelGGL(rms_scale_kernel, dim3(1), dim3(256), 0, stream, x,
                       layer->experts.hidden, eps, xscale);
  LayerCall c{};
  c.L = layer;
  c.x = x;
  c.xscale = norm_input ? xscale : nullptr;
  c.out = out;
  c.eps = eps;
  c.ids_out = ids_out;
  c.weights_out = weights_out;
  c.sg_out = sg_out;
  return run_layer(c, w8, lw, stream);
}

size_t moe_stack_workspace_bytes(const moe_layer* layers, int n_layers) {
  if (!layers || n_layers < 1 || check_layer(&layers[0]) != MOE_OK) return 0;
  return LayerWs::make(layers[0].experts.hidden, layers[0].experts.inter, layers[0].n_experts,
                       layers[0].top_k, true).total;
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
  uint8_t* w8 = reinterpret_cast<uint8_t*>(ws);
  float* xscale = reinterpret_cast<float*>(w8 + lw.xscale);
  float* xbuf = reinterpret_cast<float*>(w8 + lw.xbuf);
  hipLaunchKernelGGL(rms_scale_kernel, dim3(1), dim3(256), 0, stream, x_in, H, eps, xscale);
  const int k = layers[0].top_k;
  for (int l = 0; l < n_layers; ++l) {
    LayerCall c{};
    c.L = &layers[l];
    c.x = l == 0 ? x_in : xbuf + (size_t)((l - 1) & 1) * H;
    c.out = l == n_layers - 1 ? x_out : xbuf + (size_t)(l & 1) * H;
    c.xscale = xscale + (l & 1);
    c.xscale_next = xscale + ((l + 1) & 1);
    c.out_norm = l == n_layers - 1 ? xn_out : nullptr;
    c.eps = eps;
    c.ids_trace = ids_trace ? ids_trace + (size_t)l * k : nullptr;
    moe_status st = run_layer(c, w8, lw, stream);
    if (st != MOE_OK) return st;
  }
  return MOE_OK;
}

moe_status moe_qgemv(const moe_qmatrix* m, const float* x, float* y, hipStream_t stream) {
  if (!m || !m->rec || !x || !y) return MOE_E_NULL;
  if (m->bits != 4 && m->bits != 2) return MOE_E_BITS;
  if (m->group != 64 || m->rows < 1 ||
      !(m->cols == 256 || m->cols == 512 || m->cols == 1024 || m->cols == 2048 ||
        m->cols == 4096))
    return MOE_E_SHAPE;
  if (!aligned16(m->rec) || !aligned16(x)) return MOE_E_ALIGN;
  const uint8_t* rec = reinterpret_cast<const uint8_t*>(m->rec);
  if (m->bits == 4)
    launch_qgemv_b<4>(rec, m->rows, m->cols, x, y, stream);
  else
    launch_qgemv_b<2>(rec, m->rows, m->cols, x, y, stream);
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

}  // extern "C"
