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
// one staging copy per XCD of the layer output and of the reduced router vector.  The SwiGLU
// outputs are written by their producers into up to kGHCopies copies (XCD x reads copy
// x mod copies), so that 256 readers do not all load the same 40 KB of memory.  Zero-filled
// once with the rest of the workspace.
//
// The router all-reduce runs in three hops: every workgroup's partial vector (257 tagged pairs)
// goes to its own XCD's level-1 area (p1); workgroup j of each XCD sums slice j over the 32
// workgroups of its XCD and publishes that to the level-2 area (g2); workgroup j of each XCD
// sums the 8 XCD partials of slice j and stages the total in its XCD's copy (l_part).
struct PersistWs {
  uint32_t* ctl;       // [0] epoch of the last completed launch
  int32_t* err;
  uint64_t* g_out;     // [4096]               layer outputs, one word per row
  uint64_t* p1;        // [8][32][9][32] pairs  per XCD, slice, pair in slice, producer
  uint64_t* g2;        // [32][9][8] pairs      per slice, pair in slice, XCD
  uint64_t* g_h;       // [copies][5 * 1024]   SwiGLU outputs of the 5 slots
  uint64_t* l_out;     // [8][4096]            per-XCD staging copies
  uint64_t* l_part;    // [8][288 pairs]       per-XCD router sums

  static constexpr size_t kCtl = 256;
  static constexpr size_t kGOut = 4096 * 8, kP1 = 8 * 32 * 9 * 32 * 16, kG2 = 32 * 9 * 8 * 16,
                          kLPart = 288 * 16;
  // one copy of the SwiGLU words, padded by 1 KB so that the copies start on different channels
  static constexpr size_t kGHCopy = 5 * 1024 * 8 + 1024, kGHCopies = 8, kGH = kGHCopies * kGHCopy;
  static constexpr size_t bytes() {
    return kCtl + kGOut + kP1 + kG2 + kGH + 8 * (kGOut + kLPart);
  }

  __host__ __device__ static PersistWs at(uint8_t* p) {
    PersistWs w;
    w.ctl = reinterpret_cast<uint32_t*>(p);
    w.err = reinterpret_cast<int32_t*>(p + 64);
    size_t o = kCtl;
    w.g_out = reinterpret_cast<uint64_t*>(p + o);   o += kGOut;
    w.p1 = reinterpret_cast<uint64_t*>(p + o);      o += kP1;
    w.g2 = reinterpret_cast<uint64_t*>(p + o);      o += kG2;
    w.g_h = reinterpret_cast<uint64_t*>(p + o);     o += kGH;
    w.l_out = reinterpret_cast<uint64_t*>(p + o);   o += 8 * kGOut;
    w.l_part = reinterpret_cast<uint64_t*>(p + o);
    return w;
  }
};

bool persist_shape_ok(const moe_layer* layers, int n_layers);
bool persist_device_ok();
moe_status persist_launch(const moe_layer* layers, int n_layers, const float* x_in, float* x_out,
                          float* xn_out, float eps, int32_t* ids_trace, uint8_t* xw_base,
                          bool plain_launch, hipStream_t stream);

}  // namespace moe
