/*
 * moe.h -- C ABI of libmoe: the decode (and batched-prefill) hot path of a
 * group-quantized mixture-of-experts FFN block on AMD Instinct MI355X (gfx950).
 *
 * The operation is the one the Flash-MoE pages describe for Qwen3.5-397B-A17B:
 *  - a router matvec over 512 experts, softmax, top-4 selection
 *    (jeongsk-2ndbrain.pages.dev Flash-MoE wiki, "Per-layer pipeline";
 *    a2a-mcp.org "What is Flash-MoE", MoE section: 4 routed experts of 512 plus
 *    one shared expert per layer);
 *  - per selected expert, 4-bit or 2-bit group-quantized dequant matvecs for
 *    gate/up/down with SwiGLU fused (a2a-mcp.org deep dives 2 and 3; the wiki's
 *    techniques 2 and 3); weight = code * scale + bias per group
 *    (blog.gillilab.com flash-moe post, group quantization section);
 *  - a weighted combine of the experts with a sigmoid-gated shared expert and
 *    the residual add in a single pass (a2a-mcp.org deep dive 3), optionally
 *    followed by a two-pass RMSNorm of the result (same section; the wiki's
 *    per-layer pipeline lists expert forward + combine + norm together).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers unless a comment says "host".
 *    Descriptor structs (moe_experts, moe_qmatrix, moe_layer) are host structs
 *    read during the call; the pointers inside them are device pointers.
 *  - The caller owns every buffer.  The library allocates nothing, keeps no
 *    pointer after a call returns and holds no mutable global state; all
 *    scratch state lives in the caller's workspace.  Behaviour depends only on
 *    the arguments (no environment variables are read).
 *  - Calls are asynchronous on `stream` and return after enqueue; buffers must
 *    stay alive until the stream reaches the call.  Calls are safe from several
 *    host threads on distinct streams with distinct workspaces.  Two calls that
 *    share a workspace must be ordered on one stream.
 *  - Workspaces must be zero-filled once before first use (for example with
 *    torch.zeros); every call leaves its counters at zero again, so a workspace
 *    can be reused, and calls can be captured into HIP graphs and replayed.
 *  - Status codes are synchronous results of host-side validation made before
 *    any HIP call, except MOE_E_HIP (a launch error reported by HIP).  Device-
 *    side errors (an expert id outside [0, n_slots)) skip that expert, write
 *    zeros for it and set *dev_err = 1 when the descriptor provides dev_err.
 *  - fp32 arithmetic throughout; NaN inputs propagate; NaN router logits are
 *    never selected.
 *
 * Weight record layout (the canonical layout is also the device layout):
 *   a matrix [R x C] is codes | scale bf16 [R][C/64] | bias bf16 [R][C/64];
 *   q4 codes u8[R][C/2], element c in byte c/2, even c in the low nibble;
 *   q2 codes u8[R][C/4], element c at bits 2*(c%4) of byte c/4;
 *   weight(r, c) = code(r, c) * scale[r][c/64] + bias[r][c/64].
 *   An expert record is gate [I x H] | up [I x H] | down [H x I]
 *   (7,077,888 bytes at q4 and 3,932,160 bytes at q2 for H=4096, I=1024,
 *   matching the ~6.75 MB and ~3.9 MB per expert the pages give).
 *
 * Supported shapes: group 64; hidden H in {1024, 2048, 4096}; intermediate I
 * in {256, 512, 1024, 2048}; experts E <= 1024; top-k 1..8; at most 8 expert
 * slots per call.  Record bases must be 16-byte aligned and slot strides a
 * multiple of 16; fp32 vectors must be 16-byte aligned.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

typedef enum moe_status {
  MOE_OK = 0,
  MOE_E_NULL = 1,      /* a required pointer is NULL */
  MOE_E_SHAPE = 2,     /* unsupported or inconsistent sizes (see above) */
  MOE_E_ALIGN = 3,     /* a pointer or stride is not 16-byte aligned */
  MOE_E_BITS = 4,      /* bits is not 4 or 2 */
  MOE_E_WORKSPACE = 5, /* workspace NULL or smaller than required */
  MOE_E_HIP = 6        /* HIP reported a launch error */
} moe_status;

/* An array of expert records of one layer (slots 0..n_slots-1, equal stride). */
typedef struct moe_experts {
  const void* base;    /* device: record of slot 0 */
  int32_t bits;        /* 4 or 2 */
  int32_t hidden;      /* H: input dim of gate/up, output dim of down */
  int32_t inter;       /* I: intermediate dim */
  int32_t group;       /* must be 64 */
  int32_t n_slots;     /* number of records (512 routed + 1 shared = 513) */
  int64_t slot_bytes;  /* stride between records, >= record size, multiple of 16 */
  int32_t* dev_err;    /* device word set to 1 on an out-of-range id, or NULL */
} moe_experts;

/* One quantized matrix record [rows x cols]. */
typedef struct moe_qmatrix {
  const void* rec;     /* device: codes | scale | bias */
  int32_t bits, rows, cols, group;
} moe_qmatrix;

/* One MoE layer: experts + router.  Slots 0..n_experts-1 are routed experts. */
typedef struct moe_layer {
  moe_experts experts;
  const float* w_router; /* device fp32 [n_experts][hidden] */
  const float* w_sg;     /* device fp32 [hidden], shared-expert gate vector, or NULL (gate 1) */
  int32_t n_experts;     /* E routed experts */
  int32_t top_k;         /* k */
  int32_t shared_slot;   /* slot index of the shared expert, or -1 for none */
  /* Optional device fp32 copy of w_router blocked by 16 columns, [hidden/16][n_experts][16]
   * (written by moe_pack_router), or NULL.  The persistent stack decode multiplies each
   * workgroup's 16 output rows by the matching 16 router columns of the next layer; from this
   * copy those columns are one contiguous 32 KiB block, from w_router they are 512 strided
   * 64-byte segments, which the memory system serves several times slower.  Only the
   * persistent stack decode reads it; its contents must equal w_router. */
  const float* w_router_cb;
} moe_layer;

const char* moe_status_string(moe_status s);

/* Library version string (host). */
const char* moe_version(void);

/*
 * Router: logits[t][e] = w_router[e] . x[t], the k largest logits (ties to the
 * lower index, descending order), their softmax probabilities renormalised
 * over the k selected (equal to a softmax over all E then renormalising), and
 * shared_gate[t] = sigmoid(w_sg . x[t]).  (Wiki "Per-layer pipeline": routing
 * logits, then softmax + top-K; a2a-mcp.org deep dive 3: sigmoid gating.)
 *   x          [T][H] fp32
 *   w_router   [E][H] fp32
 *   w_sg       [H] fp32 or NULL (then shared_gate is not written)
 *   ids        [T][ld_ids] int32, columns 0..k-1 written; ld_ids >= k
 *   weights    [T][k] fp32
 *   shared_gate[T] fp32 or NULL
 *   ws         workspace of moe_router_workspace_bytes(T, E) bytes
 */
size_t moe_router_workspace_bytes(int T, int E);
moe_status moe_router_topk(const float* x, int T, const float* w_router, const float* w_sg,
                           int H, int E, int k, int32_t* ids, int ld_ids, float* weights,
                           float* shared_gate, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Expert FFNs for one token: for slot j < n, with e = ids[j] (device array),
 *   g = deq(W_gate[e]) x, u = deq(W_up[e]) x, h = silu(g) * u, y[j] = deq(W_down[e]) h.
 * (a2a-mcp.org deep dives 2-3: dequant matvec, fused SwiGLU.)
 *   x      [H] fp32;  ids [n] int32 device;  n in 1..8
 *   y      [n][H] fp32 output
 *   h      [n][I] fp32, receives the SwiGLU activations (required)
 * The _q4 / _q2 entry points require w->bits to be 4 / 2.
 */
moe_status moe_expert_ffn_q4(const moe_experts* w, const float* x, const int32_t* ids, int n,
                             float* y, float* h, hipStream_t stream);
moe_status moe_expert_ffn_q2(const moe_experts* w, const float* x, const int32_t* ids, int n,
                             float* y, float* h, hipStream_t stream);

/*
 * Combine: out = residual + sum_{j<k} weights[j] * y[j] + g * y[k], where
 * g = *shared_gate (device scalar) or 1 when shared_gate is NULL.  When
 * out_norm is not NULL it also receives out / sqrt(mean(out^2) + eps)
 * (two-pass RMSNorm, unit gain).  (a2a-mcp.org deep dive 3.)
 *   residual [H], y [k+1][H] (row k = shared expert), weights [k] device,
 *   out [H] (may alias residual), out_norm [H] or NULL.
 */
moe_status moe_combine(const float* residual, const float* y, const float* weights, int k,
                       const float* shared_gate, float* out, float* out_norm, float eps, int H,
                       hipStream_t stream);

/*
 * One MoE layer for one token, fused: router + top-k (+ shared gate), gate/up
 * + SwiGLU for the k routed experts and the shared expert, down + weighted
 * combine + residual.  With norm_input != 0 the router and experts see
 * RMSNorm(x) (unit gain, eps) while the residual is x; otherwise they see x.
 *   x [H]; out [H] (must not alias x);
 *   ids_out [k+1] / weights_out [k] / sg_out [1]: optional copies of the
 *   routing decision (device, may be NULL).
 */
size_t moe_layer_workspace_bytes(const moe_layer* layer);
moe_status moe_layer_decode(const moe_layer* layer, const float* x, int norm_input, float eps,
                            float* out, int32_t* ids_out, float* weights_out, float* sg_out,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * The same layer step for T tokens at once (small-batch decode, T in 1..64): every token is
 * routed, combined and normalised exactly as moe_layer_decode does for it alone (the pages check
 * their dequant kernel at several batch sizes: a2a-mcp.org "What is Flash-MoE", deep dive 2), and
 * gets bitwise the same result; the router and shared-expert rows are read once for all tokens.
 *   x, out [T][H] (must not overlap); ids_out [T][k (+1 with a shared slot)], weights_out
 *   [T][k], sg_out [T]: optional copies of the routing decisions.
 *   ws: moe_layer_batch_workspace_bytes(layer, T) bytes (0 for an invalid layer or T).
 * Errors: MOE_E_SHAPE for T outside 1..64 or out overlapping x, MOE_E_ALIGN for x or out not
 * 16-byte aligned, MOE_E_WORKSPACE for a short workspace, plus moe_layer_decode's layer checks.
 */
size_t moe_layer_batch_workspace_bytes(const moe_layer* layer, int T);
moe_status moe_layer_decode_batch(const moe_layer* layer, const float* x, int T, int norm_input,
                                  float eps, float* out, int32_t* ids_out, float* weights_out,
                                  float* sg_out, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * One token through a stack of layers (wiki "Per-layer pipeline": every layer
 * ends with expert forward + combine + norm).  Layer L consumes
 * RMSNorm(x_L) (unit gain, eps) and produces x_{L+1} = x_L + MoE_L(RMSNorm(x_L)).
 *   layers      host array [n_layers] of descriptors (all with equal H, I,
 *               bits, E, k)
 *   x_in  [H]   x_0;  x_out [H] = x_{n_layers};
 *   xn_out [H]  RMSNorm(x_out) or NULL; may alias x_in (x_in is only read by
 *               layer 0), which makes back-to-back calls an autoregressive loop
 *   ids_trace   [n_layers][k] int32 or NULL: routed ids chosen per layer
 *   flags       execution choice for this call (no state is kept between calls):
 *               MOE_STACK_AUTO runs the persistent kernel where the shape and the
 *               device allow it, else three kernels per layer; MOE_STACK_KERNELS
 *               always runs three kernels per layer; MOE_STACK_PERSISTENT returns
 *               MOE_E_SHAPE where the persistent kernel cannot run.  OR-ing in
 *               MOE_STACK_PLAIN_LAUNCH issues the persistent kernel with an ordinary
 *               launch instead of a cooperative one (for tracing tools that cannot
 *               follow cooperative launches): on an otherwise idle device its 256
 *               one-per-CU workgroups are still co-resident; if they are not, its
 *               bounded waits report a timeout through dev_err.  Any other bit set
 *               returns MOE_E_SHAPE.
 * Execution: for q4 or q2 layers (all of one width) of the Qwen3.5-397B-A17B block
 * shape (H 4096, I 1024, E 512, top-4, a shared expert, w_sg given) on a device with
 * 256 CUs in 8 XCDs,
 * one cooperative launch decodes up to 64 layers (persistent workgroups that
 * exchange the layer input, the logits and the SwiGLU outputs in-kernel);
 * otherwise each layer runs as three kernels.  The persistent kernel bounds
 * every wait (200 ms) and reports a timeout (bit 2) or an unexpected
 * workgroup-to-XCD placement (bit 4) by OR-ing into layers[0].experts.dev_err
 * when given; its outputs are then undefined.  The workspace must not be used
 * by two calls that can overlap.
 */
enum {
  MOE_STACK_AUTO = 0,
  MOE_STACK_KERNELS = 1,
  MOE_STACK_PERSISTENT = 2,
  MOE_STACK_PLAIN_LAUNCH = 16
};
size_t moe_stack_workspace_bytes(const moe_layer* layers, int n_layers);
moe_status moe_decode_stack(const moe_layer* layers, int n_layers, const float* x_in,
                            float* x_out, float* xn_out, float eps, int32_t* ids_trace,
                            int flags, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * T tokens (1..64) through a stack of layers at once, each exactly as moe_decode_stack with
 * MOE_STACK_KERNELS decodes it alone (three kernels per layer, bitwise the same per token):
 *   x_in, x_out [T][H] (must not overlap); xn_out [T][H] or NULL (RMSNorm of x_out, may alias
 *   x_in); ids_trace [n_layers][T][k] or NULL.
 *   ws: moe_stack_batch_workspace_bytes(layers, n_layers, T) bytes (0 for invalid arguments).
 * Errors: MOE_E_SHAPE for T outside 1..64, layers of different shapes or overlapping x_in /
 * xn_out with x_out, MOE_E_ALIGN, MOE_E_WORKSPACE, plus each layer's checks.
 */
size_t moe_stack_batch_workspace_bytes(const moe_layer* layers, int n_layers, int T);
moe_status moe_decode_stack_batch(const moe_layer* layers, int n_layers, const float* x_in,
                                  int T, float* x_out, float* xn_out, float eps,
                                  int32_t* ids_trace, void* ws, size_t ws_bytes,
                                  hipStream_t stream);

/*
 * moe_decode_stack without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, flags, results and errors as moe_decode_stack; the scratch it needs lives in
 * a 2 MiB device array inside the library, one per GPU, held until the process ends.
 *  - The first call on a device resolves that GPU's array and zero-fills it with a small
 *    kernel on `stream`, ahead of the decode.  Make that first call outside graph capture if the
 *    runtime refuses a symbol lookup during capture.
 *  - No hipMalloc / hipFree or other allocation happens in any call.
 *  - Every call on one GPU shares that GPU's array and keeps its last contents (the persistent
 *    kernel's exchange epochs continue from call to call).  Calls that can overlap on one GPU
 *    (several streams, several host threads) race on it and must be serialised by the caller.
 *  - MOE_E_WORKSPACE if the stack's workspace (moe_stack_workspace_bytes) exceeds 2 MiB (never
 *    for the supported shapes); MOE_E_HIP if the array cannot be resolved on the device.
 *  - After a reported device error (dev_err) the array's exchange state is undefined.
 */
moe_status moe_decode_stack_static(const moe_layer* layers, int n_layers, const float* x_in,
                                   float* x_out, float* xn_out, float eps, int32_t* ids_trace,
                                   int flags, hipStream_t stream);

/*
 * Batched prefill through one q4 layer (T tokens): for every token the same math as
 * moe_layer_decode with norm_input = 0 (router logits, top-k, renormalised weights,
 * sigmoid shared gate, SwiGLU expert FFNs, weighted combine + residual).  The
 * (token, expert) pairs are sorted by expert and each expert's rows run as one grouped
 * dequant GEMM on MFMA; outputs are gathered back per token.  The pages describe
 * single-token decode only; this is the batched form of the same per-token result.
 *   x [T][H], out [T][H]; ids_out [T][k], weights_out [T][k], sg_out [T]: optional
 *   (NULL allowed) copies of the routing decision.
 *   Requires bits 4, H a multiple of 512, I a multiple of 256, E a multiple of 64.
 *   ws: moe_prefill_workspace_bytes(layer, T) bytes (0 when the shape is unsupported).
 */
size_t moe_prefill_workspace_bytes(const moe_layer* layer, int T);
moe_status moe_prefill_q4(const moe_layer* layer, const float* x, int T, float* out,
                          int32_t* ids_out, float* weights_out, float* sg_out, void* ws,
                          size_t ws_bytes, hipStream_t stream);

/* Building blocks for tests. */

/*
 * Column-blocked copy of a router for moe_layer.w_router_cb:
 * dst[c][e][j] = w_router[e][16 c + j] for c < hidden / 16, e < n_experts, j < 16.
 * Both device fp32 with n_experts * hidden elements, 16-byte aligned, not overlapping;
 * hidden must be a multiple of 16 and n_experts >= 1.  A layout of the same numbers for the
 * memory system; the product it serves is the routing-logit matvec that precedes softmax +
 * top-K in the wiki's "Per-layer pipeline" (CMD2 "routing", then the CPU softmax + topK step).
 */
moe_status moe_pack_router(const float* w_router, int n_experts, int hidden, float* dst,
                           hipStream_t stream);

/*
 * y = deq(W) x for one quantized matrix; x [cols], y [rows] fp32, every weight
 * code * scale + bias of its 64-element group (blog.gillilab.com flash-moe post,
 * group quantization section; a2a-mcp.org deep dive 2).  rows >= 1; cols one of
 * 256, 512, 1024, 2048, 4096, 8192; group 64; bits 4 or 2 (else MOE_E_SHAPE /
 * MOE_E_BITS).  The record and x must be 16-byte aligned (MOE_E_ALIGN).  Besides
 * the expert matrices this serves the dense q4 attention output projection that
 * runs before the router in the same command buffer (the wiki's "Per-layer
 * pipeline", CMD2): 64 heads of 128 values (the wiki's technique 4)
 * give 8192 inputs, projected to the 4096-wide hidden state.
 */
moe_status moe_qgemv(const moe_qmatrix* m, const float* x, float* y, hipStream_t stream);

/*
 * Standalone two-pass RMSNorm with unit gain over T rows of H:
 * out[t] = x[t] / sqrt(mean(x[t]^2) + eps) (a2a-mcp.org deep dive 3: a sum-of-
 * squares reduction, then the scaling pass; the wiki's "Per-layer pipeline" puts a
 * norm between o_proj and the router).  x, out [T][H] fp32 device; out may equal x
 * (in place), any other overlap is undefined.  T >= 1 and H >= 1 (MOE_E_SHAPE).
 * One workgroup per row.
 */
moe_status moe_rmsnorm(const float* x, int T, int H, float eps, float* out,
                       hipStream_t stream);

/*
 * GatedDeltaNet state update for one decoded token, in place.  The wiki (jeongsk-2ndbrain.pages.dev
 * Flash-MoE, technique 4, "Accelerate BLAS linear attention") updates 64 heads of 128 x 128 fp32 state per
 * linear-attention layer with a scale, a matrix-vector product and a rank-one update per head;
 * the pages print no formula, and this is the published gated delta rule (Yang, Kautz and
 * Hatamizadeh, "Gated Delta Networks") in its one-token form.  Per head h:
 *   S_h <- alpha[h] * S_h;  u = S_h k_h;  S_h <- S_h + beta[h] * (v_h - u) k_h^T;  out_h = S_h q_h
 *   state [n_heads][dv][dk] fp32, row i of a head indexed by value, column j by key (updated in
 *   place); q, k [n_heads][dk]; v, out [n_heads][dv]; alpha, beta [n_heads]; all device fp32.
 * dk must be 128 and dv a multiple of 8 (>= 8), n_heads >= 1, n_heads * dv <= 2^24
 * (MOE_E_SHAPE); state, q and k 16-byte aligned (MOE_E_ALIGN).  out must not overlap the other
 * buffers.  Gating values are taken as given (any decay, any beta); q and k are not normalised
 * here.
 */
moe_status moe_gdn_step(float* state, const float* q, const float* k, const float* v,
                        const float* alpha, const float* beta, int n_heads, int dk, int dv,
                        float* out, hipStream_t stream);

/*
 * Copy n canonical expert records laid out back to back at `canonical` into
 * slots [slot0, slot0+n) of the resident array described by `dst` (stride
 * dst->slot_bytes).  The pages treat each expert as one record that is read
 * whole (a2a-mcp.org "What is Flash-MoE", deep dive 1, and the wiki's technique 1:
 * about 6.75 MB per 4-bit expert; the damoang.net post's SSD paragraph: about
 * 3.9 MB per expert at 2 bits); the record here is gate | up | down, each codes |
 * scale | bias, which gives exactly those sizes.  The canonical layout is the
 * device layout, so packing is a strided copy.
 *   canonical  device, n * record bytes, 16-byte aligned (MOE_E_ALIGN)
 *   dst        descriptor of the resident slots (validated as for the decode calls);
 *              0 <= slot0, slot0 + n <= dst->n_slots, n >= 1 (MOE_E_SHAPE)
 * The source and destination must not overlap.
 */
moe_status moe_pack(const void* canonical, int n, int slot0, const moe_experts* dst,
                    hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
