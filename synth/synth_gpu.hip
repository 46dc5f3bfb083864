// synth_gpu.hip -- device side of the seeded synthetic-input generator.
//
// Fills expert records directly in device memory with exactly the bytes that
// synth_cpu.c writes on the host (both use the draw definitions of synth.h).
// A full 60-layer stack is ~218 GB, far too much to generate on the host and
// copy, so weights are generated where they live.  Test/benchmark input only.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "synth.h"

namespace {

// one thread per 64-bit draw of codes
__global__ void fill_codes_kernel(uint8_t* __restrict__ base, uint64_t slot_bytes, int slot0,
                                  int nslots, uint64_t mat_off, uint64_t nwords, uint64_t seed,
                                  int layer, int tensor) {
  uint64_t gid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint64_t total = nwords * (uint64_t)nslots;
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t t = gid; t < total; t += stride) {
    uint64_t s = t / nwords;
    uint64_t w = t - s * nwords;
    uint64_t key = synth_key(seed, (uint64_t)layer, (uint64_t)(slot0 + s), (uint64_t)tensor);
    uint64_t d = synth_draw(key, w);
    uint64_t* dst = reinterpret_cast<uint64_t*>(base + s * slot_bytes + mat_off) + w;
    *dst = d;
  }
}

// one thread per (scale, bias) pair
__global__ void fill_meta_kernel(uint8_t* __restrict__ base, uint64_t slot_bytes, int slot0,
                                 int nslots, uint64_t scale_off, uint64_t nmeta, uint64_t seed,
                                 int layer, int tensor, double lo, double hi, double zp) {
  uint64_t gid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint64_t total = nmeta * (uint64_t)nslots;
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t t = gid; t < total; t += stride) {
    uint64_t s = t / nmeta;
    uint64_t i = t - s * nmeta;
    uint64_t key = synth_key(seed, (uint64_t)layer, (uint64_t)(slot0 + s), (uint64_t)tensor);
    uint16_t sc = synth_scale_bf16(synth_draw(key, i), lo, hi);
    uint16_t* sp = reinterpret_cast<uint16_t*>(base + s * slot_bytes + scale_off);
    sp[i] = sc;
    sp[nmeta + i] = synth_bias_bf16(sc, zp);
  }
}

int launch_matrix(uint8_t* base, uint64_t slot_bytes, int slot0, int nslots, uint64_t mat_off,
                  int bits, int R, int C, int G, uint64_t seed, int layer, int codes_tensor,
                  int scale_tensor, double lo, double hi, double zp, hipStream_t st) {
  uint64_t ncode = synth_codes_bytes(bits, R, C);
  uint64_t nmeta = synth_meta_count(R, C, G);
  const int threads = 256;
  const unsigned blocks = 8192;
  hipLaunchKernelGGL(fill_codes_kernel, dim3(blocks), dim3(threads), 0, st, base, slot_bytes,
                     slot0, nslots, mat_off, ncode / 8, seed, layer, codes_tensor);
  if (hipGetLastError() != hipSuccess) return 1;
  hipLaunchKernelGGL(fill_meta_kernel, dim3(blocks), dim3(threads), 0, st, base, slot_bytes,
                     slot0, nslots, mat_off + ncode, nmeta, seed, layer, scale_tensor, lo, hi, zp);
  if (hipGetLastError() != hipSuccess) return 1;
  return 0;
}

}  // namespace

extern "C" {

// Fill expert slots [slot0, slot0 + nslots) of one layer.  base points at slot
// 0 of the layer's expert array; consecutive slots are slot_bytes apart.
// Returns 0 on success, nonzero on a bad argument or launch failure.
int synth_gpu_fill_experts(void* base, uint64_t slot_bytes, int slot0, int nslots, uint64_t seed,
                           int layer, int bits, int H, int I, int G, double lo, double hi, double zp,
                           void* stream) {
  if (!base || nslots <= 0 || (bits != 4 && bits != 2) || G <= 0 || H % G || I % G) return 2;
  if ((H * bits) % 64 || (I * bits) % 64) return 2;  // code rows are whole 64-bit words
  if (slot_bytes < synth_expert_bytes(bits, H, I, G) || slot_bytes % 8) return 2;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  uint8_t* b = reinterpret_cast<uint8_t*>(base);
  uint64_t mg = synth_matrix_bytes(bits, I, H, G);
  int rc = 0;
  rc |= launch_matrix(b, slot_bytes, slot0, nslots, 0, bits, I, H, G, seed, layer,
                      SYNTH_T_GATE_CODES, SYNTH_T_GATE_SCALE, lo, hi, zp, st);
  rc |= launch_matrix(b, slot_bytes, slot0, nslots, mg, bits, I, H, G, seed, layer,
                      SYNTH_T_UP_CODES, SYNTH_T_UP_SCALE, lo, hi, zp, st);
  rc |= launch_matrix(b, slot_bytes, slot0, nslots, 2 * mg, bits, H, I, G, seed, layer,
                      SYNTH_T_DOWN_CODES, SYNTH_T_DOWN_SCALE, lo, hi, zp, st);
  return rc;
}

}  // extern "C"
