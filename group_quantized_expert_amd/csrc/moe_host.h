// moe_host.h -- host-side validation and workspace layout helpers of libmoe.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr size_t kAlign = 256;
constexpr int kDownRows = 16;  // output rows per block of the down kernel

inline size_t align_up(size_t v, size_t a = kAlign) { return (v + a - 1) / a * a; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

inline bool hidden_ok(int H) { return H == 1024 || H == 2048 || H == 4096; }
inline bool inter_ok(int I) { return I == 256 || I == 512 || I == 1024 || I == 2048; }

inline int64_t matrix_bytes(int bits, int R, int C) {
  return (int64_t)R * C * bits / 8 + 4 * (int64_t)R * (C / 64);
}
inline int64_t expert_bytes(int bits, int H, int I) {
  return 2 * matrix_bytes(bits, I, H) + matrix_bytes(bits, H, I);
}

inline moe_status check_experts(const moe_experts* w) {
  if (!w || !w->base) return MOE_E_NULL;
  if (w->bits != 4 && w->bits != 2) return MOE_E_BITS;
  if (w->group != 64 || !hidden_ok(w->hidden) || !inter_ok(w->inter) || w->n_slots < 1)
    return MOE_E_SHAPE;
  if (w->slot_bytes < expert_bytes(w->bits, w->hidden, w->inter)) return MOE_E_SHAPE;
  if (!aligned16(w->base) || (w->slot_bytes % 16) != 0) return MOE_E_ALIGN;
  return MOE_OK;
}

inline moe_status check_layer(const moe_layer* L) {
  if (!L) return MOE_E_NULL;
  moe_status st = check_experts(&L->experts);
  if (st != MOE_OK) return st;
  if (!L->w_router) return MOE_E_NULL;
  if (L->n_experts < 1 || L->n_experts > 1024 || L->top_k < 1 || L->top_k > 8 ||
      L->top_k > L->n_experts || L->n_experts > L->experts.n_slots)
    return MOE_E_SHAPE;
  if (L->shared_slot >= L->experts.n_slots || L->shared_slot < -1) return MOE_E_SHAPE;
  if (!aligned16(L->w_router) || (L->w_sg && !aligned16(L->w_sg)) ||
      (L->w_router_cb && !aligned16(L->w_router_cb)))
    return MOE_E_ALIGN;
  return MOE_OK;
}

// Digit planes of a decode input for the gate/up products: per 32 inputs a record of
// kDigPlanes planes and one (input sum, digit unit) word, 16 bytes each.
constexpr int kDigPlanes = 7;
constexpr int kDigRec = kDigPlanes + 1;  // 16-byte words per record

// Workspace of one decode layer for T tokens (also the per-layer part of the stack workspace):
// router logits [T][E], ids [T][k + 1], weights [T][k], shared gates [T], SwiGLU outputs
// [T][k + 1][I], the inputs' digit-plane records [T][H / 32][kDigRec] and RMS scales [T] and,
// for a stack, an input/output ping-pong [2][T][H].
struct LayerWs {
  size_t logits, ids, weights, sg, h, xdig, xscale, xbuf, total;
  static LayerWs make(int H, int I, int E, int k, bool stack, int T = 1) {
    LayerWs w{};
    const size_t t = (size_t)T;
    size_t o = 0;
    w.logits = o;    o = align_up(o + t * E * sizeof(float));
    w.ids = o;       o = align_up(o + t * (k + 1) * sizeof(int32_t));
    w.weights = o;   o = align_up(o + t * k * sizeof(float));
    w.sg = o;        o = align_up(o + t * sizeof(float));
    w.h = o;         o = align_up(o + t * (k + 1) * I * sizeof(float));
    w.xdig = o;      o = align_up(o + t * (size_t)(H / 32) * kDigRec * 16);
    w.xscale = o;    o = align_up(o + t * sizeof(float));
    w.xbuf = o;      if (stack) o = align_up(o + 2 * t * H * sizeof(float));
    w.total = o;
    return w;
  }
};

}  // namespace moe
