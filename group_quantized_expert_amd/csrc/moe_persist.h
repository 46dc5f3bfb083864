// moe_persist.h -- host interface of the persistent stack decode kernel (moe_persist.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kPersistMaxLayers = 64;   // layers per launch (longer stacks are split)
constexpr int kPersistErrTimeout = 2;   // dev_err bits set by the persistent kernel
constexpr int kPersistErrPlacement = 4;

// Exchange area inside the stack workspace: control words, the global tagged buffers and
// one staging copy per XCD.  Zero-filled once with the rest of the workspace.
struct PersistWs {
  uint32_t* ctl;       // [0] epoch of the last completed launch
  int32_t* err;
  uint64_t* g_out;     // [4096]
  uint64_t* g_logit;   // [512]
  uint64_t* g_h;       // [5 * 1024]
  uint64_t* l_out;     // [8][4096]
  uint64_t* l_logit;   // [8][512]
  uint64_t* l_h;       // [8][5 * 1024]

  static constexpr size_t kCtl = 256;
  static constexpr size_t kGOut = 4096 * 8, kGLogit = 512 * 8, kGH = 5 * 1024 * 8;
  static constexpr size_t bytes() { return kCtl + 9 * (kGOut + kGLogit + kGH); }

  __host__ __device__ static PersistWs at(uint8_t* p) {
    PersistWs w;
    w.ctl = reinterpret_cast<uint32_t*>(p);
    w.err = reinterpret_cast<int32_t*>(p + 64);
    size_t o = kCtl;
    w.g_out = reinterpret_cast<uint64_t*>(p + o);   o += kGOut;
    w.g_logit = reinterpret_cast<uint64_t*>(p + o); o += kGLogit;
    w.g_h = reinterpret_cast<uint64_t*>(p + o);     o += kGH;
    w.l_out = reinterpret_cast<uint64_t*>(p + o);   o += 8 * kGOut;
    w.l_logit = reinterpret_cast<uint64_t*>(p + o); o += 8 * kGLogit;
    w.l_h = reinterpret_cast<uint64_t*>(p + o);
    return w;
  }
};

bool persist_shape_ok(const moe_layer* layers, int n_layers);
bool persist_device_ok();
moe_status persist_launch(const moe_layer* layers, int n_layers, const float* x_in, float* x_out,
                          float* xn_out, float eps, int32_t* ids_trace, uint8_t* xw_base,
                          hipStream_t stream);

}  // namespace moe
