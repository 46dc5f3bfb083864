// GatedDeltaNet state update for one decoded token (moe_gdn_step).
//
// The linear-attention layers keep per head a 128 x 128 fp32 state and update it each token with
// a scale, a matrix-vector product and a rank-one update (Flash-MoE wiki, technique 4,
// "Accelerate BLAS linear attention": 64 heads; a2a-mcp.org deep dive 4).  Read as the gated
// delta rule, per head h and state row i (value index):
//   s_i <- alpha_h s_i;  u_i = s_i . k_h;  s_i <- s_i + beta_h (v_hi - u_i) k_h;  o_hi = s_i . q_h
// Every row is independent given k, q, v, alpha and beta, so the update is one pass over the
// state: each row is read once, updated in registers and written back in place, and its read-out
// is reduced from the same registers.  The pass is bound by HBM: 2 * 512 bytes per row.
//
// Work split: a 32-lane half-wave owns one row (a float4 per lane); a wave owns 8 consecutive
// rows (4 passes of 2), whose loads are all issued before the first is used.  dv is a multiple
// of 8, so a wave's rows share one head and k, q, alpha, beta are loaded once per wave.  The
// state is streamed (read once, written once per token), so its loads and stores carry the
// nontemporal hint.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"
#include "moe_device.h"
#include "moe_host.h"

namespace moe {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGdnDk = 128;
constexpr int kGdnRowsPerWave = 8;
constexpr int kGdnBlock = 256;

__device__ __forceinline__ float dot4(const float4 a, const float4 b) {
  return fmaf(a.w, b.w, fmaf(a.z, b.z, fmaf(a.y, b.y, a.x * b.x)));
}

__global__ __launch_bounds__(kGdnBlock) void gdn_step_kernel(float* S, const float* q,
                                                             const float* k, const float* v,
                                                             const float* alpha,
                                                             const float* beta, int dv, int rows,
                                                             float* o) {
  const int lane = threadIdx.x & (kWave - 1);
  const int half = lane >> 5, l = lane & 31;
  const int wave = blockIdx.x * (kGdnBlock / kWave) + (threadIdx.x / kWave);
  const int r0 = wave * kGdnRowsPerWave;
  if (r0 >= rows) return;  // no block-wide synchronisation below
  const int h = r0 / dv;
  float4* srow = reinterpret_cast<float4*>(S) + (size_t)r0 * (kGdnDk / 4) + l;
  float4 st[kGdnRowsPerWave / 2];
#pragma unroll
  for (int p = 0; p < kGdnRowsPerWave / 2; ++p) {
    const f32x4 t = __builtin_nontemporal_load(
        reinterpret_cast<const f32x4*>(&srow[(size_t)(2 * p + half) * (kGdnDk / 4)]));
    st[p] = make_float4(t[0], t[1], t[2], t[3]);
  }
  const float4 kk = reinterpret_cast<const float4*>(k + (size_t)h * kGdnDk)[l];
  const float4 qq = reinterpret_cast<const float4*>(q + (size_t)h * kGdnDk)[l];
  const float a = alpha[h], b = beta[h];
  float vv[kGdnRowsPerWave / 2];
#pragma unroll
  for (int p = 0; p < kGdnRowsPerWave / 2; ++p) vv[p] = v[r0 + 2 * p + half];
#pragma unroll
  for (int p = 0; p < kGdnRowsPerWave / 2; ++p) {
    float4 s = st[p];
    s.x *= a;
    s.y *= a;
    s.z *= a;
    s.w *= a;
    const float u = seg_sum<32>(dot4(s, kk));
    const float d = b * (vv[p] - u);
    s.x = fmaf(d, kk.x, s.x);
    s.y = fmaf(d, kk.y, s.y);
    s.z = fmaf(d, kk.z, s.z);
    s.w = fmaf(d, kk.w, s.w);
    const f32x4 t = {s.x, s.y, s.z, s.w};
    __builtin_nontemporal_store(t, reinterpret_cast<f32x4*>(&srow[(size_t)(2 * p + half) * (kGdnDk / 4)]));
    const float on = seg_sum<32>(dot4(s, qq));
    if (l == 0) o[r0 + 2 * p + half] = on;
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_gdn_step(float* state, const float* q, const float* k, const float* v,
                                   const float* alpha, const float* beta, int n_heads, int dk,
                                   int dv, float* out, hipStream_t stream) {
  if (!state || !q || !k || !v || !alpha || !beta || !out) return MOE_E_NULL;
  if (n_heads < 1 || dk != kGdnDk || dv < kGdnRowsPerWave || dv % kGdnRowsPerWave ||
      (int64_t)n_heads * dv > (1 << 24))
    return MOE_E_SHAPE;
  if (!aligned16(state) || !aligned16(q) || !aligned16(k)) return MOE_E_ALIGN;
  const int rows = n_heads * dv;
  const int waves = rows / kGdnRowsPerWave;
  const int blocks = (waves + kGdnBlock / kWave - 1) / (kGdnBlock / kWave);
  hipLaunchKernelGGL(gdn_step_kernel, dim3(blocks), dim3(kGdnBlock), 0, stream, state, q, k, v,
                     alpha, beta, dv, rows, out);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_E_HIP;
}
